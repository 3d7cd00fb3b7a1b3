// Fused piecewise attention for fp32 inputs (d = 64 or 128), plain fp32 FMA on the vector ALUs.
// Same three phases and the same online-softmax state as the bf16 kernel (gist.science summary
// of the PISA paper, section 2 "Core algorithm" and "Hardware implementation").
//
// One workgroup per (head, query block); D/32 adjacent threads share a query row, each owning
// 32 of its dimensions (q, accumulator). Scores are reduced across those threads with shuffles,
// so every thread of a row holds the row's full softmax state (max m, sum l, beta).
// Phase 2 keeps the pages' form: e = 2^{s log2e scale - m}, l += n_j e, beta += e, O += e sumV_j,
// with the shift m covering s + log2 n_j.
#include "dev_common.h"
#include "pisa_internal.h"

namespace pisa {
namespace {

constexpr int kMaskWords = (8192 + 128) / 32;

template <int TPR>
__device__ __forceinline__ float row_reduce(float x) {
  x += __shfl_xor(x, 1);
  if (TPR == 4) x += __shfl_xor(x, 2);
  return x;
}

template <int D, int BLK>
__global__ __launch_bounds__(BLK * (D / 32)) void attend_f32(Dims dm, Work w, const float* __restrict__ Q,
                                                             const float* __restrict__ K,
                                                             const float* __restrict__ V,
                                                             float* __restrict__ out) {
  constexpr int TPR = D / 32, NTH = BLK * TPR, CH = 16;
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
  const int c0 = 32 * sub;

  float q[32], O[32];
  for (int c = 0; c < 32; ++c) {
    q[c] = row < n_i ? Q[head + (size_t)(i * B + row) * D + c0 + c] : 0.f;
    O[c] = 0.f;
  }
  const int nmask = (dm.Nbp + 31) / 32;
  for (int t = tid; t < nmask; t += NTH) selm[t] = 0u;
  __syncthreads();
  const int32_t* sel = w.idx + ((size_t)h * Nb + i) * kk;
  for (int t = tid; t < kk; t += NTH) atomicOr(&selm[sel[t] >> 5], 1u << (sel[t] & 31));

  const float cs = dm.scale * kLog2e;
  float m = -INFINITY, l = 0.f, beta = 0.f;

  // ---- phase 1 ----
  for (int it = 0; it < kk; ++it) {
    const int j = sel[it];
    const int n_j = (j == Nb - 1) ? dm.n_last : B;
    __syncthreads();
    for (int e = tid; e < BLK * D; e += NTH) {
      const int r = e / D;
      const size_t g = head + (size_t)j * B * D + e;
      Ks[e] = r < n_j ? K[g] : 0.f;
      Vs[e] = r < n_j ? V[g] : 0.f;
    }
    __syncthreads();
    for (int n0 = 0; n0 < BLK; n0 += CH) {
      float s[CH];
      float mx = -INFINITY;
#pragma unroll 2
      for (int x = 0; x < CH; ++x) {
        float part = 0.f;
        for (int c = 0; c < 32; ++c) part = fmaf(q[c], Ks[(n0 + x) * D + c0 + c], part);
        const float full = row_reduce<TPR>(part);
        s[x] = (n0 + x < n_j) ? full * cs : -INFINITY;
        mx = fmaxf(mx, s[x]);
      }
      const float m_new = fmaxf(m, mx);
      const float alpha = m == m_new ? 1.0f : exp2f(m - m_new);
      m = m_new;
      l *= alpha;
      beta *= alpha;
      for (int c = 0; c < 32; ++c) O[c] *= alpha;
#pragma unroll 2
      for (int x = 0; x < CH; ++x) {
        const float p = exp2f(s[x] - m);
        l += p;
        for (int c = 0; c < 32; ++c) O[c] = fmaf(p, Vs[(n0 + x) * D + c0 + c], O[c]);
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
      for (int e = tid; e < BLK * D; e += NTH) {
        const int r = e / D;
        const bool ok = cb + r < Nb;
        Ks[e] = ok ? kb[(size_t)cb * D + e] : 0.f;
        Vs[e] = ok ? vs[(size_t)cb * D + e] : 0.f;
      }
      __syncthreads();
      for (int n0 = 0; n0 < BLK; n0 += CH) {
        float s[CH];
        float mx = -INFINITY;
#pragma unroll 2
        for (int x = 0; x < CH; ++x) {
          const int j = cb + n0 + x;
          float part = 0.f;
          for (int c = 0; c < 32; ++c) part = fmaf(q[c], Ks[(n0 + x) * D + c0 + c], part);
          const float full = row_reduce<TPR>(part);
          const bool ok = j < Nb && !((selm[j >> 5] >> (j & 31)) & 1u);
          s[x] = ok ? full * cs : -INFINITY;
          mx = fmaxf(mx, s[x] + (j == Nb - 1 ? lgLast : lgB));
        }
        const float m_new = fmaxf(m, mx);
        const float alpha = m == m_new ? 1.0f : exp2f(m - m_new);
        m = m_new;
        l *= alpha;
        beta *= alpha;
        for (int c = 0; c < 32; ++c) O[c] *= alpha;
#pragma unroll 2
        for (int x = 0; x < CH; ++x) {
          const int j = cb + n0 + x;
          const float e = exp2f(s[x] - m);
          const float nj = (j == Nb - 1) ? (float)dm.n_last : (float)B;
          l = fmaf(e, nj, l);
          beta += e;
          for (int c = 0; c < 32; ++c) O[c] = fmaf(e, Vs[(n0 + x) * D + c0 + c], O[c]);
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
    for (int e = tid; e < D * D; e += NTH) Hs[e] = hb[e];
    for (int c = 0; c < 32; ++c) Qs[row * D + c0 + c] = q[c];
    __syncthreads();
    const float bs = beta * dm.scale;
#pragma unroll 1
    for (int c = 0; c < 32; ++c) {
      float t = 0.f;
      for (int a = 0; a < D; ++a) t = fmaf(Qs[row * D + a], Hs[a * D + c0 + c], t);
      O[c] = fmaf(bs, t, O[c]);
    }
  }

  if (row < n_i) {
    const float inv = 1.0f / l;
    float* o = out + head + (size_t)(i * B + row) * D + c0;
    for (int c = 0; c < 32; ++c) o[c] = O[c] * inv;
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
  hipLaunchKernelGGL((attend_f32<D, BLK>), dim3(items), dim3(BLK * (D / 32)), 0, s, dm, w, q, k, v, o)
  if (dm.d == 64 && dm.B == 64) PISA_F32(64, 64);
  else if (dm.d == 64) PISA_F32(64, 128);
  else if (dm.B == 64) PISA_F32(128, 64);
  else PISA_F32(128, 128);
#undef PISA_F32
  return hipGetLastError();
}

}  // namespace pisa
