// Fused piecewise attention for fp32 inputs (d = 64 or 128), plain fp32 FMA on the vector ALUs.
// Same three phases and the same online-softmax state as the bf16 kernel (gist.science summary
// of the PISA paper, section 2 "Core algorithm" and "Hardware implementation").
//
// One workgroup per (head, query block); 8 adjacent threads share a query row, each owning D/8
// of its dimensions (q, accumulator), so that a key's dot product is a short chain per thread.
// Scores are reduced across those threads with DPP lane moves, so every thread of a row holds the
// row's full softmax state (max m, sum l, beta). Tiles move in 16-byte pieces.
// Phase 2 keeps the pages' form: e = 2^{s log2e scale - m}, l += n_j e, beta += e, O += e sumV_j,
// with the shift m covering s + log2 n_j.
#include "dev_common.h"
#include "pisa_internal.h"

namespace pisa {
namespace {

constexpr int kMaskWords = (8192 + 128) / 32;

// Sum over the 8 adjacent lanes (aligned) that share a row, on DPP lane moves: the neighbour in
// the quad (quad_perm 1,0,3,2), the other pair of the quad (2,3,0,1), then the other quad of the
// 8 lanes (row_half_mirror maps lane i to 7 - i). Every lane of the 8 ends with the same sum.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_reduce8(float x) {
  x += dpp_move<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp_move<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp_move<0x141>(x);  // row_half_mirror
  return x;
}

// NA tiles of rows x D floats from global (row stride D) into LDS, 16 bytes per load, all of the
// thread's loads in flight before the first store; rows >= valid read as 0
template <int D, int ROWS, int NTH, int NA = 1>
__device__ __forceinline__ void tiles_in(float* const (&dst)[NA], const float* const (&src)[NA], int valid, int tid) {
  constexpr int kAll = ROWS * D / 4, kPer = (kAll + NTH - 1) / NTH;
  f32x4 v[NA][kPer];
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e4 = tid + NTH * u;
      const bool ok = e4 < kAll && (4 * e4) / D < valid;
      v[a][u] = ok ? *reinterpret_cast<const f32x4*>(src[a] + 4 * e4) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e4 = tid + NTH * u;
      if (e4 < kAll) *reinterpret_cast<f32x4*>(dst[a] + 4 * e4) = v[a][u];
    }
}

template <int D, int BLK>
__global__ __launch_bounds__(BLK * 8) void attend_f32(Dims dm, Work w, const float* __restrict__ Q,
                                                             const float* __restrict__ K,
                                                             const float* __restrict__ V,
                                                             float* __restrict__ out) {
  constexpr int TPR = 8, DPT = D / TPR, NTH = BLK * TPR, CH = 16;  // row_reduce8: TPR = 8
  constexpr int LDSF = (2 * BLK * D > D * D + BLK * D) ? 2 * BLK * D : D * D + BLK * D;
  __shared__ __attribute__((aligned(16))) float smem[LDSF];
  __shared__ uint32_t selm[kMaskWords];
  float* Ks = smem;
  float* Vs = smem + BLK * D;

  const int item = blockIdx.x;
  const int h = item / dm.Nb, i = item % dm.Nb;
  const int tid = threadIdx.x, row = tid / TPR, sub = tid % TPR;
  const int Nb = dm.Nb, B = dm.B, kk = dm.k;
  const int n_i = (i == Nb - 1) ? dm.n_last : B;
  const size_t head = (size_t)h * dm.L * D;
  const int c0 = DPT * sub;

  float q[DPT], O[DPT];
#pragma unroll
  for (int c4 = 0; c4 < DPT / 4; ++c4) {
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (row < n_i) v = *reinterpret_cast<const f32x4*>(Q + head + (size_t)(i * B + row) * D + c0 + 4 * c4);
#pragma unroll
    for (int e = 0; e < 4; ++e) q[4 * c4 + e] = v[e];
  }
#pragma unroll
  for (int c = 0; c < DPT; ++c) O[c] = 0.f;
  const int nmask = (dm.Nbp + 31) / 32;
  for (int t = tid; t < nmask; t += NTH) selm[t] = 0u;
  __syncthreads();
  const int32_t* sel = w.idx + ((size_t)h * Nb + i) * kk;
  for (int t = tid; t < kk; t += NTH) atomicOr(&selm[sel[t] >> 5], 1u << (sel[t] & 31));

  const float cs = dm.scale * kLog2e;
  float m = -INFINITY, l = 0.f, beta = 0.f;

  // ---- phase 1 ----
  // The next block's K and V are loaded into registers (this thread's 16-byte pieces) while the
  // current block is used, where the registers allow (up to 64 x 128 or 128 x 64 floats a tile).
  constexpr int kPer = BLK * D / 4 / NTH;
  constexpr bool kPrefetch = BLK * D <= 8192;
  f32x4 pk[kPrefetch ? kPer : 1], pv[kPrefetch ? kPer : 1];
  auto fetch = [&](int it) __attribute__((always_inline)) {
    const int j = sel[it];
    const int n_j = (j == Nb - 1) ? dm.n_last : B;
    const float* kb = K + head + (size_t)j * B * D;
    const float* vb = V + head + (size_t)j * B * D;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e4 = tid + NTH * u;
      const bool ok = (4 * e4) / D < n_j;
      pk[u] = ok ? *reinterpret_cast<const f32x4*>(kb + 4 * e4) : f32x4{0.f, 0.f, 0.f, 0.f};
      pv[u] = ok ? *reinterpret_cast<const f32x4*>(vb + 4 * e4) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  if constexpr (kPrefetch) {
    if (kk > 0) fetch(0);
  }
  for (int it = 0; it < kk; ++it) {
    const int j = sel[it];
    const int n_j = (j == Nb - 1) ? dm.n_last : B;
    __syncthreads();
    if constexpr (kPrefetch) {
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int e4 = tid + NTH * u;
        *reinterpret_cast<f32x4*>(Ks + 4 * e4) = pk[u];
        *reinterpret_cast<f32x4*>(Vs + 4 * e4) = pv[u];
      }
    } else {
      tiles_in<D, BLK, NTH, 2>({Ks, Vs}, {K + head + (size_t)j * B * D, V + head + (size_t)j * B * D}, n_j, tid);
    }
    __syncthreads();
    if constexpr (kPrefetch) {
      if (it + 1 < kk) fetch(it + 1);
      // keep the loads here: the scheduler would otherwise sink them to their use a block later
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int n0 = 0; n0 < BLK; n0 += CH) {
      float s[CH];
      float mx = -INFINITY;
#pragma unroll 2
      for (int x = 0; x < CH; ++x) {
        float part = 0.f;
#pragma unroll
        for (int c = 0; c < DPT; ++c) part = fmaf(q[c], Ks[(n0 + x) * D + c0 + c], part);
        const float full = row_reduce8(part);
        s[x] = (n0 + x < n_j) ? full * cs : -INFINITY;
        mx = fmaxf(mx, s[x]);
      }
      const float m_new = fmaxf(m, mx);
      const float alpha = m == m_new ? 1.0f : exp2f(m - m_new);
      m = m_new;
      l *= alpha;
      beta *= alpha;
#pragma unroll
      for (int c = 0; c < DPT; ++c) O[c] *= alpha;
#pragma unroll 2
      for (int x = 0; x < CH; ++x) {
        const float p = exp2f(s[x] - m);
        l += p;
#pragma unroll
        for (int c = 0; c < DPT; ++c) O[c] = fmaf(p, Vs[(n0 + x) * D + c0 + c], O[c]);
      }
    }
  }

  const bool do_tail = kk < Nb && (dm.phases & 2);
  // ---- phase 2 ----
  if (do_tail) {
    const float* kb = w.kbar + (size_t)h * Nb * D;
    const float* vs = w.vsum + (size_t)h * Nb * D;
    const float lgB = log2f((float)B), lgLast = log2f((float)dm.n_last);
    for (int cb = 0; cb < dm.Nbp; cb += BLK) {
      __syncthreads();
      tiles_in<D, BLK, NTH, 2>({Ks, Vs}, {kb + (size_t)cb * D, vs + (size_t)cb * D}, Nb - cb, tid);
      __syncthreads();
      for (int n0 = 0; n0 < BLK; n0 += CH) {
        float s[CH];
        float mx = -INFINITY;
#pragma unroll 2
        for (int x = 0; x < CH; ++x) {
          const int j = cb + n0 + x;
          float part = 0.f;
#pragma unroll
          for (int c = 0; c < DPT; ++c) part = fmaf(q[c], Ks[(n0 + x) * D + c0 + c], part);
          const float full = row_reduce8(part);
          const bool ok = j < Nb && !((selm[j >> 5] >> (j & 31)) & 1u);
          s[x] = ok ? full * cs : -INFINITY;
          mx = fmaxf(mx, s[x] + (j == Nb - 1 ? lgLast : lgB));
        }
        const float m_new = fmaxf(m, mx);
        const float alpha = m == m_new ? 1.0f : exp2f(m - m_new);
        m = m_new;
        l *= alpha;
        beta *= alpha;
#pragma unroll
        for (int c = 0; c < DPT; ++c) O[c] *= alpha;
#pragma unroll 2
        for (int x = 0; x < CH; ++x) {
          const int j = cb + n0 + x;
          const float e = exp2f(s[x] - m);
          const float nj = (j == Nb - 1) ? (float)dm.n_last : (float)B;
          l = fmaf(e, nj, l);
          beta += e;
#pragma unroll
          for (int c = 0; c < DPT; ++c) O[c] = fmaf(e, Vs[(n0 + x) * D + c0 + c], O[c]);
        }
      }
    }
  }

  // ---- phase 3 ----
  if (do_tail && (dm.phases & 4)) {
    float* Hs = smem;
    float* Qs = smem + D * D;
    __syncthreads();
    const float* hb = w.hbar + (size_t)h * D * D;
    tiles_in<D, D, NTH>({Hs}, {hb}, D, tid);
#pragma unroll
    for (int c = 0; c < DPT; ++c) Qs[row * D + c0 + c] = q[c];
    __syncthreads();
    const float bs = beta * dm.scale;
#pragma unroll 1
    for (int c = 0; c < DPT; ++c) {
      float t = 0.f;
#pragma unroll 8
      for (int a = 0; a < D; ++a) t = fmaf(Qs[row * D + a], Hs[a * D + c0 + c], t);
      O[c] = fmaf(bs, t, O[c]);
    }
  }

  if (row < n_i) {
    const float inv = 1.0f / l;
    float* o = out + head + (size_t)(i * B + row) * D + c0;
#pragma unroll
    for (int c4 = 0; c4 < DPT / 4; ++c4)
      *reinterpret_cast<f32x4*>(o + 4 * c4) =
          f32x4{O[4 * c4] * inv, O[4 * c4 + 1] * inv, O[4 * c4 + 2] * inv, O[4 * c4 + 3] * inv};
  }
}

}  // namespace

hipError_t launch_attend_f32(const Dims& dm, const Work& w, const void* Q, const void* K, const void* V, void* out,
                             hipStream_t s) {
  const int items = dm.H * dm.Nb;
  auto q = static_cast<const float*>(Q);
  auto k = static_cast<const float*>(K);
  auto v = static_cast<const float*>(V);
  auto o = static_cast<float*>(out);
#define PISA_F32(D, BLK) \
  hipLaunchKernelGGL((attend_f32<D, BLK>), dim3(items), dim3(BLK * 8), 0, s, dm, w, q, k, v, o)
  if (dm.d == 64 && dm.B == 64) PISA_F32(64, 64);
  else if (dm.d == 64) PISA_F32(64, 128);
  else if (dm.B == 64) PISA_F32(128, 64);
  else PISA_F32(128, 128);
#undef PISA_F32
  return hipGetLastError();
}

}  // namespace pisa
