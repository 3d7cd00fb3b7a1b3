// Routing: for every query block i of a head, Score_{i,j} over all key blocks j and the top-k
// critical set S_i (gist.science summary of the PISA paper, section 2 "Covariance-aware
// routing": the score combines the attention score with the block covariance norm M_j; the AI
// Radio episode names the per-block score Score_{t,j}). The score is
//   covariance-aware: qbar_i . kbar_j + ln(n_j + ||qbar_i||_2 M_j)
//   plain:            qbar_i . kbar_j
// in fp32 with a fixed summation order (c = 0..d-1). Selection keeps the k largest scores, ties
// to the smaller j, and writes S_i as ascending block indices.
//
// One workgroup = 4 waves = 16 query blocks of one head; wave w owns 4 rows. Key-block centroids
// stream through LDS in tiles of 64 (lane = block within the tile) and are shared by the 16 rows.
// Each lane keeps the scores of blocks j = 64 s + lane in registers as order-preserving uint32
// keys; the k-th largest key is found MSB-first with wave ballots (32 rounds), then the blocks
// are compacted in ascending j with ballot/popcount prefix sums.
#include "dev_common.h"
#include "pisa_internal.h"

namespace pisa {
namespace {

// RPW query blocks per wave (4 waves): fewer for large N_b so that the RPW x NS keys stay in
// registers.
template <int D, int NS, int RPW>
__global__ __launch_bounds__(256) void route_kernel(Dims dm, Work w) {
  constexpr int kRows = 4 * RPW;
  constexpr int kRowsPerWave = RPW;
  constexpr int STR = D + 4;  // padded row stride (floats) of the LDS tiles
  __shared__ __attribute__((aligned(16))) float qs[kRows][STR];
  __shared__ __attribute__((aligned(16))) float kt[64][STR];
  __shared__ float qn[kRows];
  const int h = blockIdx.y, i0 = blockIdx.x * kRows;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int Nb = dm.Nb;
  const float* qbar = w.qbar + (size_t)h * Nb * D;
  const float* kbar = w.kbar + (size_t)h * Nb * D;
  const float* M = w.M + (size_t)h * Nb;

#pragma unroll
  for (int e = tid; e < kRows * D; e += 256) {  // all loads in flight at once
    const int r = e / D, c = e % D;
    qs[r][c] = (i0 + r < Nb) ? qbar[(size_t)(i0 + r) * D + c] : 0.f;
  }
  __syncthreads();
  if (tid < kRows) {
    float s = 0.f;
    for (int c = 0; c < D; ++c) s = fmaf(qs[tid][c], qs[tid][c], s);
    qn[tid] = sqrtf(s);
  }

  // key[][] is indexed with compile-time indices only (every loop over it is unrolled), so that it
  // stays in registers
  uint32_t key[kRowsPerWave][NS];
  // The next centroid tile (this thread's share, and M_j of the lane's key) is loaded into
  // registers while the current one is used, so one tile's load latency overlaps the previous
  // tile's dot products instead of adding up load by load.
  constexpr int kPer = 64 * (D / 4) / 256;  // 16-byte pieces of a tile per thread
  f32x4 pre[kPer];
  float mpre = 0.f;
  auto fetch = [&](int jt) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < kPer; ++it) {
      const int e = tid + 256 * it;
      const int r = e / (D / 4), c4 = e % (D / 4);
      pre[it] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (jt + r < Nb) pre[it] = *reinterpret_cast<const f32x4*>(kbar + (size_t)(jt + r) * D + 4 * c4);
    }
    mpre = (jt + lane < Nb) ? M[jt + lane] : 0.f;
  };
  fetch(0);
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    __syncthreads();  // previous tile consumed (and qn visible on the first pass)
    const int jt = 64 * s;
    float mj = 0.f;
    if (jt < Nb) {
#pragma unroll
      for (int it = 0; it < kPer; ++it) {
        const int e = tid + 256 * it;
        const int r = e / (D / 4), c4 = e % (D / 4);
        *reinterpret_cast<f32x4*>(&kt[r][4 * c4]) = pre[it];
      }
      mj = mpre;
      if (jt + 64 < Nb) fetch(jt + 64);
    }
    __syncthreads();
    const int j = jt + lane;
    float acc[kRowsPerWave];
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) acc[r] = 0.f;
    if (jt < Nb) {
      for (int c4 = 0; c4 < D / 4; ++c4) {
        const f32x4 kv = *reinterpret_cast<const f32x4*>(&kt[lane][4 * c4]);
#pragma unroll
        for (int r = 0; r < kRowsPerWave; ++r) {
          const f32x4 qv = *reinterpret_cast<const f32x4*>(&qs[kRowsPerWave * wave + r][4 * c4]);
          acc[r] = fmaf(qv[0], kv[0], acc[r]);
          acc[r] = fmaf(qv[1], kv[1], acc[r]);
          acc[r] = fmaf(qv[2], kv[2], acc[r]);
          acc[r] = fmaf(qv[3], kv[3], acc[r]);
        }
      }
    }
    const bool valid = j < Nb;
    const float nj = (j == Nb - 1) ? (float)dm.n_last : (float)dm.B;
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
      float sc = acc[r];
      if (dm.routing == 0) sc += logf(fmaf(qn[kRowsPerWave * wave + r], mj, nj));
      key[r][s] = valid ? float_order_key(sc) : 0u;
    }
  }

  const uint64_t ltmask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int kk = dm.k;
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
    const int i = i0 + kRowsPerWave * wave + r;
    if (i >= Nb) break;  // uniform per wave
    uint32_t T = 0;
    for (int b = 31; b >= 0; --b) {
      const uint32_t cand = T | (1u << b);
      int cnt = 0;
#pragma unroll
      for (int s = 0; s < NS; ++s) cnt += __popcll(__ballot(key[r][s] >= cand));
      if (cnt >= kk) T = cand;
    }
    int gt = 0;
#pragma unroll
    for (int s = 0; s < NS; ++s) gt += __popcll(__ballot(key[r][s] > T));
    const int need = kk - gt;
    int eq_seen = 0, base = 0;
    int32_t* out = w.idx + ((size_t)h * Nb + i) * kk;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bool eq = key[r][s] == T;
      const uint64_t eqm = __ballot(eq);
      const bool take = key[r][s] > T || (eq && eq_seen + __popcll(eqm & ltmask) < need);
      eq_seen += __popcll(eqm);
      const uint64_t sm = __ballot(take);
      if (take) out[base + __popcll(sm & ltmask)] = 64 * s + lane;
      base += __popcll(sm);
    }
  }
}

}  // namespace

hipError_t launch_route(const Dims& dm, const Work& w, hipStream_t s) {
  const int ns = (dm.Nb + 63) / 64;
#define PISA_ROUTE(D, NS, RPW)                                                             \
  hipLaunchKernelGGL((route_kernel<D, NS, RPW>), dim3((dm.Nb + 4 * RPW - 1) / (4 * RPW), dm.H), \
                     dim3(256), 0, s, dm, w)
  if (dm.d == 128) {
    if (ns <= 4) PISA_ROUTE(128, 4, 4);
    else if (ns <= 12) PISA_ROUTE(128, 12, 4);
    else if (ns <= 16) PISA_ROUTE(128, 16, 4);
    else if (ns <= 32) PISA_ROUTE(128, 32, 2);
    else PISA_ROUTE(128, 128, 1);
  } else {
    if (ns <= 4) PISA_ROUTE(64, 4, 4);
    else if (ns <= 16) PISA_ROUTE(64, 16, 4);
    else if (ns <= 32) PISA_ROUTE(64, 32, 2);
    else PISA_ROUTE(64, 128, 1);
  }
#undef PISA_ROUTE
  return hipGetLastError();
}

}  // namespace pisa
