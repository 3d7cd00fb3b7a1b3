// Routing: for every query block i of a head, Score_{i,j} over all key blocks j and the top-k
// critical set S_i (gist.science summary of the PISA paper, section 2 "Covariance-aware
// routing": the score combines the attention score with the block covariance norm M_j; the AI
// Radio episode names the per-block score Score_{t,j}). The score is
//   covariance-aware: qbar_i . kbar_j + ln(n_j + ||qbar_i||_2 M_j)
//   plain:            qbar_i . kbar_j
// in fp32 with a fixed summation order (c = 0..d-1). Selection keeps the k largest scores, ties
// to the smaller j, and writes S_i as ascending block indices.
//
// One workgroup = 4 waves = 16 query blocks of one head (fewer for N_b > 1024); wave w selects
// the rows 4w .. 4w + 3. d = 128 with 16 rows: the scores run on the fp32 matrix unit, each wave
// taking 16 keys of every tile of 64 into registers straight from memory (one tile ahead), and
// land as order-preserving uint32 keys in a per-workgroup LDS array; the waves meet once, then
// select. Otherwise key-block centroids stream through LDS in tiles of 64 (lane = block within
// the tile), shared by the rows, with fp32 FMA dot products, and every lane keeps its keys in
// registers. The k-th largest key is found MSB-first with wave ballots, then the blocks are
// compacted in ascending j with ballot/popcount prefix sums.
#include "dev_common.h"
#include "pisa_internal.h"

namespace pisa {
namespace {

// RPW query blocks per wave (4 waves): fewer for large N_b so that the RPW x NS keys stay in
// registers.
// Radix select of one row's k largest keys and their compaction: lane l holds the keys of blocks
// j = 64 s + l (0 for j >= N_b); writes the k selected j in ascending order to out.
template <int NS>
__device__ __forceinline__ void select_row(const uint32_t (&key)[NS], int Nb, int kk, int lane, int32_t* out) {
  const uint64_t ltmask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // Every valid key lies between the row's smallest and largest, so all of them share the bits
  // above the highest bit where those two differ: the k-th largest has them too, and the select
  // starts below them (the same T as starting at bit 31, in fewer rounds).
  uint32_t kmax = 0u, kmin = 0xffffffffu;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const bool valid = 64 * s + lane < Nb;
    kmax = max(kmax, valid ? key[s] : 0u);
    kmin = min(kmin, valid ? key[s] : 0xffffffffu);
  }
  for (int o = 32; o >= 1; o >>= 1) {
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
  }
  kmax = __builtin_amdgcn_readfirstlane(kmax);
  kmin = __builtin_amdgcn_readfirstlane(kmin);
  const uint32_t diff = kmax ^ kmin;
  const int top = diff ? 31 - __builtin_clz(diff) : -1;  // highest differing bit
  // the shared prefix above `top` (all of kmax when every key is equal)
  uint32_t T = top < 0 ? kmax : (top == 31 ? 0u : (kmax & ~((2u << top) - 1u)));
  for (int b = top; b >= 0; --b) {
    const uint32_t cand = T | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int s = 0; s < NS; ++s) cnt += __popcll(__ballot(key[s] >= cand));
    if (cnt >= kk) T = cand;
    // exactly k keys at or above cand: they are the k largest, whatever the lower bits decide
    if (cnt == kk) break;
  }
  int gt = 0;
#pragma unroll
  for (int s = 0; s < NS; ++s) gt += __popcll(__ballot(key[s] > T));
  const int need = kk - gt;
  int eq_seen = 0, base = 0;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const bool eq = key[s] == T;
    const uint64_t eqm = __ballot(eq);
    const bool take = key[s] > T || (eq && eq_seen + __popcll(eqm & ltmask) < need);
    eq_seen += __popcll(eqm);
    const uint64_t sm = __ballot(take);
    if (take) out[base + __popcll(sm & ltmask)] = 64 * s + lane;
    base += __popcll(sm);
  }
}

// RPW query blocks per wave (4 waves): fewer for large N_b so that the RPW x NS keys stay in
// registers.
template <int D, int NS, int RPW>
__global__ __launch_bounds__(256) void route_kernel(Dims dm, Work w) {
  constexpr int kRows = 4 * RPW;
  constexpr int kRowsPerWave = RPW;
  // 16 query blocks per workgroup at d = 128: scores on the matrix unit; otherwise fp32 FMA
  constexpr bool kMatrix = D == 128 && kRows == 16;
  constexpr int STR = D + 4;  // padded row stride (floats) of the LDS tiles
  __shared__ __attribute__((aligned(16))) float qs[kRows][STR];
  const int h = blockIdx.y, i0 = blockIdx.x * kRows;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int Nb = dm.Nb;
  const float* qbar = w.qbar + (size_t)h * Nb * D;
  const float* kbar = w.kbar + (size_t)h * Nb * D;
  const float* M = w.M + (size_t)h * Nb;
  const int kk = dm.k;

  {
    // the workgroup's pooled queries, 16 bytes per load, all in flight at once; rows past N_b
    // read as zeros (buffer range check)
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qbar + (size_t)i0 * D, (uint32_t)max(0, Nb - i0) * D * 4);
    constexpr int kAll = kRows * D / 4;                 // 16-byte pieces
    constexpr int kPieces = (kAll + 255) / 256;         // per thread (the last round partial)
    f32x4 qv[kPieces];
#pragma unroll
    for (int it = 0; it < kPieces; ++it)
      if (tid + 256 * it < kAll) qv[it] = __builtin_bit_cast(f32x4, buf_load16(rq, 16u * (tid + 256 * it)));
#pragma unroll
    for (int it = 0; it < kPieces; ++it) {
      const int e = 4 * (tid + 256 * it);
      if (tid + 256 * it < kAll) *reinterpret_cast<f32x4*>(&qs[e / D][e % D]) = qv[it];
    }
  }
  __syncthreads();

  if constexpr (kMatrix) {
    // Scores on the fp32 matrix unit (v_mfma_f32_16x16x4_f32): rows = the workgroup's 16 query
    // blocks, columns = 16 keys per wave and tile of 64. The sum over d runs as 32 steps of 4
    // with lane l covering d = 32 (l / 16) + t at step t (A: row l % 16, B: key l % 16), so each
    // lane's operands are 32 consecutive floats of one row. Lane l then holds the scores of rows
    // 4 (l / 16) .. + 3 for its key. They go to the workgroup's score array as order-preserving
    // keys (rows KS floats apart, KS = 4 mod 64: the 64 lanes' writes fall in distinct banks), and
    // the waves run through their tiles without meeting; one barrier ends the pass, then each
    // wave selects its rows from the array.
    constexpr int KS = 64 * NS + 4;
    __shared__ uint32_t sk[16][KS];
    float qa[32];
    {
      const float* qrow = &qs[lane & 15][32 * (lane >> 4)];
#pragma unroll
      for (int t4 = 0; t4 < 8; ++t4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(qrow + 4 * t4);
#pragma unroll
        for (int e = 0; e < 4; ++e) qa[4 * t4 + e] = v[e];
      }
    }
    // ||qbar|| of the rows this lane's scores belong to, 4 (l / 16) + r, from the operands: each
    // lane sums the squares of its 32 values (d ascending), then the four lane groups of a row
    // are added (groups 0 + 1, 2 + 3, then the two pairs)
    float qn[4];
    {
      float ss = 0.f;
#pragma unroll
      for (int t = 0; t < 32; ++t) ss = fmaf(qa[t], qa[t], ss);
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      const float nrm = sqrtf(ss);
#pragma unroll
      for (int r = 0; r < 4; ++r) qn[r] = __shfl(nrm, 4 * (lane >> 4) + r);
    }
    // The centroids of tile s + 1 are loaded while tile s is used, through buffer resources that
    // end at N_b: keys past it read as zeros, and every tile issues the same loads, so the wait
    // before a tile's use counts only the younger tile's loads.
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbar, (uint32_t)Nb * D * 4);
    const __amdgpu_buffer_rsrc_t rm = make_rsrc(M, (uint32_t)Nb * 4);
    f32x4 kb[8], kpre[8];
    float mpre;
    auto fetch = [&](int jt) __attribute__((always_inline)) {
      const uint32_t jk = jt + 16 * wave + (lane & 15);
      const uint32_t off = jk * (D * 4) + 128u * (lane >> 4);
#pragma unroll
      for (int t4 = 0; t4 < 8; ++t4) kpre[t4] = __builtin_bit_cast(f32x4, buf_load16(rk, off + 16u * t4));
      mpre = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rm, 4u * jk, 0, 0));
    };
    fetch(0);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int jt = 64 * s;
#pragma unroll
      for (int t4 = 0; t4 < 8; ++t4) kb[t4] = kpre[t4];
      const float mj = mpre;
      if (s + 1 < NS) fetch(jt + 64);
      // keep the loads here: the scheduler would otherwise sink them to their use a tile later
      __builtin_amdgcn_sched_barrier(0);
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 32; ++t) c = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[t], kb[t >> 2][t & 3], c, 0, 0, 0);
      const int jk = jt + 16 * wave + (lane & 15);
      const float nj = (jk == Nb - 1) ? (float)dm.n_last : (float)dm.B;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float sc = c[r];
        if (dm.routing == 0) sc += logf(fmaf(qn[r], mj, nj));
        sk[4 * (lane >> 4) + r][jk] = jk < Nb ? float_order_key(sc) : 0u;
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
      const int i = i0 + kRowsPerWave * wave + r;
      if (i >= Nb) break;  // uniform per wave
      uint32_t key[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s) key[s] = sk[kRowsPerWave * wave + r][64 * s + lane];
      select_row<NS>(key, Nb, kk, lane, w.idx + ((size_t)h * Nb + i) * kk);
    }
  } else {
    __shared__ float qn[kRows];
    if (tid < kRows) {
      float s2 = 0.f;
      for (int c = 0; c < D; ++c) s2 = fmaf(qs[tid][c], qs[tid][c], s2);
      qn[tid] = sqrtf(s2);
    }
    // key[][] is indexed with compile-time indices only (every loop over it is unrolled), so that
    // it stays in registers
    uint32_t key[kRowsPerWave][NS];
    __shared__ __attribute__((aligned(16))) float kt[64][STR];
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
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
      const int i = i0 + kRowsPerWave * wave + r;
      if (i >= Nb) break;  // uniform per wave
      select_row<NS>(key[r], Nb, kk, lane, w.idx + ((size_t)h * Nb + i) * kk);
    }
  }
}

}  // namespace

hipError_t launch_route(const Dims& dm, const Work& w, hipStream_t s) {
  const int ns = (dm.Nb + 63) / 64;
#define PISA_ROUTE(D, NS, RPW)                                                             \
  hipLaunchKernelGGL((route_kernel<D, NS, RPW>), dim3((dm.Nb + 4 * RPW - 1) / (4 * RPW), dm.H), \
                     dim3(256), 0, s, dm, w)
  if (dm.d == 128) {  // the tile count rounded up to an even number up to 12 (no idle tiles)
    if (ns <= 2) PISA_ROUTE(128, 2, 4);
    else if (ns <= 4) PISA_ROUTE(128, 4, 4);
    else if (ns <= 6) PISA_ROUTE(128, 6, 4);
    else if (ns <= 8) PISA_ROUTE(128, 8, 4);
    else if (ns <= 10) PISA_ROUTE(128, 10, 4);
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
