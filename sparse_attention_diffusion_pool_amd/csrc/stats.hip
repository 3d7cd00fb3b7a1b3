// Block statistics for PISA (the precompute step of the fused kernel described on the
// gist.science summary of the PISA paper, section 2 "Hardware implementation"; the statistics
// themselves follow section 2 "Core algorithm" - centroid and value sum of every block - and
// "Covariance-aware routing" - the block first-order matrices H_j, their mean H-bar and
// M_j = ||H_j - H-bar||).
//
// Pass A (one workgroup per 16 consecutive blocks of a head): column sums of Q, K, V per block
// (pooled scaled query, key centroid, value sum) and the partial sum of the block first-order
// matrices over its blocks, H_j = K_j^T V_j - kbar_j (sum V_j)^T (= sum_n (k_n - kbar_j)^T v_n).
// Finalize (per head): H-bar = (sum of the partials) / N_b; bf16 copies of the pooled tokens and
// of H-bar^T for the attention kernel. Covariance pass (one workgroup per block): H_j again, then
// M_j = ||H_j - H-bar||_F (and H_j^T in bf16 for the block-wise first-order variant).
//
// bf16 inputs: K_j^T V_j on v_mfma_f32_32x32x16_bf16 (products of bf16 values are exact in fp32,
// accumulation fp32); both operands come from row-major LDS tiles through ds_read_b64_tr_b16.
// fp32 inputs: plain fp32 FMA.
#include "dev_common.h"
#include "pisa_internal.h"

namespace pisa {
namespace {

__device__ __forceinline__ void unpack_bf16x8(u32x4 x, float* f) {
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(x[i] << 16);
    f[2 * i + 1] = __uint_as_float(x[i] & 0xffff0000u);
  }
}

// K^T V of one B x 128 block held in two transpose-read LDS tiles; wave w owns rows 32w..32w+31
// of the 128 x 128 product: acc[ct] covers columns 32ct..32ct+31.
template <int BLK>
__device__ __forceinline__ void ktv_mfma(const char* Ks, const char* Vs, f32x16 acc[4], int wave, int lane) {
  const uint32_t hh = lane >> 5, g16 = (lane >> 4) & 1, l16 = lane & 15;
#pragma unroll
  for (int ks = 0; ks < BLK / 16; ++ks) {
    const uint32_t klo = 16 * ks + 8 * hh;
    bf16x8 a = tr_operand(Ks, klo, klo + 4, 32 * wave + 16 * g16, l16);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      bf16x8 b = tr_operand(Vs, klo, klo + 4, 32 * ct + 16 * g16, l16);
      acc[ct] = mfma32(a, b, acc[ct]);
    }
  }
}

// The same product, plus the block's column sums on the matrix unit: ksum = K^T 1 (the K^T operand
// against a ones operand) and vsum = 1^T V for the wave's own 32 columns. Products with 1.0 are
// exact and the sums accumulate in fp32. Rows past the block end are zero in the tiles.
// Lane l holds: ksum[x] = column sum of K for d = 32 wave + 8 (x >> 2) + 4 (l >> 5) + (x & 3);
// vsum[0] = column sum of V for column 32 wave + (l & 31).
template <int BLK>
__device__ __forceinline__ void ktv_mfma_sums(const char* Ks, const char* Vs, f32x16 acc[4], f32x16& ksum,
                                              f32x16& vsum, int wave, int lane) {
  const uint32_t hh = lane >> 5, g16 = (lane >> 4) & 1, l16 = lane & 15;
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
  ksum = f32x16{};
  vsum = f32x16{};
#pragma unroll
  for (int ks = 0; ks < BLK / 16; ++ks) {
    const uint32_t klo = 16 * ks + 8 * hh;
    const bf16x8 a = tr_operand(Ks, klo, klo + 4, 32 * wave + 16 * g16, l16);
    ksum = mfma32(a, ones, ksum);
    const bf16x8 bw = tr_operand(Vs, klo, klo + 4, 32 * wave + 16 * g16, l16);
    vsum = mfma32(ones, bw, vsum);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const bf16x8 b = tr_operand(Vs, klo, klo + 4, 32 * ct + 16 * g16, l16);
      acc[ct] = mfma32(a, b, acc[ct]);
    }
  }
}

// Pass A, bf16. One LDS stage (64 KB) and two workgroups per CU: each workgroup copies a block's K
// and V tiles to LDS (Q rows into registers), then sums and multiplies them, while the other
// workgroup on the CU has its block in flight. (Two stages in one workgroup would keep only one
// block in flight per CU: LDS holds about two blocks.) The chunk's partial is corrected by the
// centroids block by block: G_c = sum_{j in c} (K_j^T V_j - kbar_j (sum V_j)^T) = sum_{j in c} H_j.
template <int BLK>
__global__ __launch_bounds__(256, 2) void stats_pass_bf16(Dims dm, Work w, const __bf16* __restrict__ Q,
                                                          const __bf16* __restrict__ K,
                                                          const __bf16* __restrict__ V) {
  __shared__ __attribute__((aligned(1024))) char Ks[BLK * 256];
  __shared__ __attribute__((aligned(1024))) char Vs[BLK * 256];
  __shared__ float red[4][128];  // per-wave column sums of Q
  __shared__ float svs[128];     // the current block's value sums
  constexpr int QR = BLK / 16;   // Q rows (16-byte pieces) per thread
  const int h = blockIdx.y, c = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j0 = c * dm.chunk, j1 = min(dm.Nb, j0 + dm.chunk);
  const size_t head = (size_t)h * dm.L * 128;
  const uint32_t hh = lane >> 5, l32 = lane & 31;
  f32x16 acc[4];
  for (int ct = 0; ct < 4; ++ct) acc[ct] = f32x16{};
  const int p = tid & 15, rg = tid >> 4;  // column chunk (8 columns) and row group for the sums
  u32x4 qa[QR];

  auto rows_of = [&](int j) { return (j == dm.Nb - 1) ? dm.n_last : dm.B; };
  for (int j = j0; j < j1; ++j) {
    const int n = rows_of(j);
    const size_t r0 = head + (size_t)j * dm.B * 128;
    tile_to_lds<true>(make_rsrc(K + r0, n * 256), 256, Ks, BLK, wave, 4, lane);
    tile_to_lds<true>(make_rsrc(V + r0, n * 256), 256, Vs, BLK, wave, 4, lane);
    {
      const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + r0, n * 256);
#pragma unroll
      for (int e = 0; e < QR; ++e) qa[e] = buf_load16(rq, (rg + 16 * e) * 256 + p * 16);
    }
    wait_vmem();
    __syncthreads();  // the block's tiles landed
    const float inv = 1.0f / (float)n;
    const size_t ob = ((size_t)h * dm.Nb + j) * 128;
    // Q (in registers): VALU sums over this thread's rows, then across the 16-lane row groups
    float qs[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < QR; ++e) {
      float f[8];
      unpack_bf16x8(qa[e], f);
      for (int x = 0; x < 8; ++x) qs[x] += f[x];
    }
    for (int x = 0; x < 8; ++x) {
      qs[x] += __shfl_xor(qs[x], 16);
      qs[x] += __shfl_xor(qs[x], 32);
    }
    if (lane < 16)
      for (int x = 0; x < 8; ++x) red[wave][8 * p + x] = qs[x];
    // K and V (in LDS): column sums on the matrix unit beside K^T V
    f32x16 ksum, vsum;
    ktv_mfma_sums<BLK>(Ks, Vs, acc, ksum, vsum, wave, lane);
    // lane l's ksum[x] is the column sum of K for row a = 32 wave + 8 (x >> 2) + 4 hh + (x & 3) of
    // the product, the same row as acc[.][x]
    if (l32 == 0) {
#pragma unroll
      for (int x = 0; x < 16; ++x) w.kbar[ob + 32 * wave + 8 * (x >> 2) + 4 * hh + (x & 3)] = ksum[x] * inv;
    }
    if (lane < 32) {
      w.vsum[ob + 32 * wave + lane] = vsum[0];
      svs[32 * wave + lane] = vsum[0];
    }
    __syncthreads();  // red and svs complete; every wave done with the tiles
    if (tid < 128) {
      const float sq = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
      w.qbar[ob + tid] = sq * dm.scale * inv;
    }
    // acc[ct][x] -= kbar_j[a] vsum_j[b], b = 32 ct + l32
    float vb[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) vb[ct] = svs[32 * ct + l32];
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const float ka = ksum[x] * inv;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) acc[ct][x] = fmaf(-ka, vb[ct], acc[ct][x]);
    }
    __syncthreads();  // red and svs read before the next block overwrites them
  }
  float* G = w.G + ((size_t)h * dm.NC + c) * 128 * 128;
  for (int ct = 0; ct < 4; ++ct)
    for (int x = 0; x < 16; ++x) {
      const int a = 32 * wave + 8 * (x >> 2) + 4 * hh + (x & 3);
      G[a * 128 + 32 * ct + l32] = acc[ct][x];
    }
}

// ---------------------------------------------------------------------------------------------
// Spectral-norm variant of M_j: the largest singular value of E = H_j - H-bar. Lanczos on E^T E
// (Krylov basis from a fixed start vector, both Gram-Schmidt passes repeated against every basis
// vector), at most kLanczos steps or until the basis spans an invariant subspace, then the largest
// eigenvalue of the Lanczos tridiagonal by 64-lane multisection on its Sturm count. E (row stride
// D + 1 floats), the basis and the scratch live in LDS; all 256 threads call it.
// ---------------------------------------------------------------------------------------------

constexpr int kLanczos = 32;

template <int D>
struct SpecLds {
  float E[D][D + 1];
  float Qb[kLanczos + 1][D + 1];  // Lanczos basis, one vector per row
  float u[D], w[D];
  float part[256 / D][D];
  float coef[kLanczos + 1];
  float alpha[kLanczos], beta[kLanczos];
  float red[4];
  float lo_hi[2];
  int m;
};

// number of eigenvalues below x of the symmetric tridiagonal (a[0..m-1], off-diagonal b[0..m-2])
__device__ __forceinline__ int sturm_count(const float* a, const float* b, int m, float x) {
  float d = a[0] - x;
  int cnt = d < 0.f;
  for (int i = 1; i < m; ++i) {
    if (d == 0.f) d = 1e-30f;
    d = a[i] - x - b[i - 1] * b[i - 1] / d;
    cnt += d < 0.f;
  }
  return cnt;
}

template <int D>
__device__ float spectral_norm(SpecLds<D>& S, int tid) {
  constexpr int TPR = 256 / D;   // threads per row / column
  constexpr int SEG = D / TPR;
  const int lane = tid & 63, wave = tid >> 6;
  auto block_sum = [&](float x) {  // sum over all 256 threads
    x = wave_sum(x);
    __syncthreads();
    if (lane == 0) S.red[wave] = x;
    __syncthreads();
    return S.red[0] + S.red[1] + S.red[2] + S.red[3];
  };
  // ||E||_F^2 sets the scale of the breakdown test; fixed start vector 1 + cos(r), normalised
  float fro = 0.f;
  for (int e = tid; e < D * D; e += 256) fro += S.E[e / D][e % D] * S.E[e / D][e % D];
  fro = block_sum(fro);
  if (!(fro > 0.f)) return 0.f;
  float q0 = 0.f;
  if (tid < D) q0 = 1.0f + __cosf((float)tid);
  const float n0 = block_sum(q0 * q0);
  if (tid < D) S.Qb[0][tid] = q0 * rsqrtf(n0);
  __syncthreads();
  const int K = D < kLanczos ? D : kLanczos;
  int m = K;
  for (int k = 0; k < K; ++k) {
    {  // u = E q_k (four independent partial sums keep several LDS reads in flight)
      const int r = tid / TPR, pt = tid % TPR;
      float a4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
      for (int c = pt * SEG; c < (pt + 1) * SEG; c += 4)
        for (int x = 0; x < 4; ++x) a4[x] = fmaf(S.E[r][c + x], S.Qb[k][c + x], a4[x]);
      float acc = (a4[0] + a4[1]) + (a4[2] + a4[3]);
      for (int o = 1; o < TPR; o <<= 1) acc += __shfl_xor(acc, o);
      if (pt == 0) S.u[r] = acc;
    }
    __syncthreads();
    {  // w = E^T u (partials over row segments)
      const int c = tid % D, pt = tid / D;
      float a4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
      for (int r = pt * SEG; r < (pt + 1) * SEG; r += 4)
        for (int x = 0; x < 4; ++x) a4[x] = fmaf(S.E[r + x][c], S.u[r + x], a4[x]);
      S.part[pt][c] = (a4[0] + a4[1]) + (a4[2] + a4[3]);
    }
    __syncthreads();
    if (tid < D) {
      float acc = 0.f;
      for (int pt = 0; pt < TPR; ++pt) acc += S.part[pt][tid];
      S.w[tid] = acc;
    }
    __syncthreads();
    float a_k = 0.f;
    for (int pass = 0; pass < 2; ++pass) {  // w -= Q (Q^T w), twice
      {
        const int i = tid / TPR, pt = tid % TPR;
        float a4[4] = {0.f, 0.f, 0.f, 0.f};
        if (i <= k) {
#pragma unroll 4
          for (int r = pt * SEG; r < (pt + 1) * SEG; r += 4)
            for (int x = 0; x < 4; ++x) a4[x] = fmaf(S.Qb[i][r + x], S.w[r + x], a4[x]);
        }
        float acc = (a4[0] + a4[1]) + (a4[2] + a4[3]);
        for (int o = 1; o < TPR; o <<= 1) acc += __shfl_xor(acc, o);
        if (pt == 0 && i <= k) S.coef[i] = acc;
      }
      __syncthreads();
      a_k += S.coef[k];
      {
        const int r = tid % D, pt = tid / D;
        float a2[2] = {0.f, 0.f};
        int i = pt;
        for (; i + TPR <= k; i += 2 * TPR) {
          a2[0] = fmaf(S.coef[i], S.Qb[i][r], a2[0]);
          a2[1] = fmaf(S.coef[i + TPR], S.Qb[i + TPR][r], a2[1]);
        }
        if (i <= k) a2[0] = fmaf(S.coef[i], S.Qb[i][r], a2[0]);
        S.part[pt][r] = a2[0] + a2[1];
      }
      __syncthreads();
      if (tid < D) {
        float acc = 0.f;
        for (int pt = 0; pt < TPR; ++pt) acc += S.part[pt][tid];
        S.w[tid] -= acc;
      }
      __syncthreads();
    }
    const float wr = tid < D ? S.w[tid] : 0.f;
    const float b_k = sqrtf(block_sum(wr * wr));
    if (tid == 0) {
      S.alpha[k] = a_k;
      S.beta[k] = b_k;
    }
    if (b_k <= 1e-6f * fro || k == K - 1) {  // invariant subspace reached (or last step)
      m = k + 1;
      break;
    }
    if (tid < D) S.Qb[k + 1][tid] = wr / b_k;
    __syncthreads();
  }
  __syncthreads();
  // largest eigenvalue of the tridiagonal: eigenvalues of E^T E lie in [0, ||E||_F^2]
  if (wave == 0) {
    float lo = 0.f, hi = fro * 1.0001f;
    for (int it = 0; it < 6; ++it) {
      const float x = lo + (hi - lo) * (float)(lane + 1) / 65.0f;
      const bool all_below = sturm_count(S.alpha, S.beta, m, x) == m;
      const uint64_t bal = __ballot(all_below);
      const int first = bal ? __builtin_ctzll(bal) : 64;
      const float nhi = first < 64 ? lo + (hi - lo) * (float)(first + 1) / 65.0f : hi;
      const float nlo = first > 0 ? lo + (hi - lo) * (float)first / 65.0f : lo;
      lo = nlo;
      hi = nhi;
    }
    if (lane == 0) {
      S.lo_hi[0] = lo;
      S.lo_hi[1] = hi;
    }
  }
  __syncthreads();
  return sqrtf(0.5f * (S.lo_hi[0] + S.lo_hi[1]));
}

// SPEC: spectral-norm M_j; HJT: also store H_j^T in bf16 (block-wise first-order variant)
template <int BLK, bool SPEC, bool HJT>
__global__ __launch_bounds__(256) void stats_cov_bf16(Dims dm, Work w, const __bf16* __restrict__ K,
                                                      const __bf16* __restrict__ V) {
  __shared__ __attribute__((aligned(1024))) char Ks[BLK * 256];
  __shared__ __attribute__((aligned(1024))) char Vs[BLK * 256];
  __shared__ float red[4];
  __shared__ SpecLds<SPEC ? 128 : 1> spec;
  const int h = blockIdx.y, j = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = (j == dm.Nb - 1) ? dm.n_last : dm.B;
  const size_t r0 = (size_t)h * dm.L * 128 + (size_t)j * dm.B * 128;
  tile_to_lds<true>(make_rsrc(K + r0, n * 256), 256, Ks, BLK, wave, 4, lane);
  tile_to_lds<true>(make_rsrc(V + r0, n * 256), 256, Vs, BLK, wave, 4, lane);
  wait_vmem();
  __syncthreads();
  f32x16 acc[4];
  for (int ct = 0; ct < 4; ++ct) acc[ct] = f32x16{};
  ktv_mfma<BLK>(Ks, Vs, acc, wave, lane);
  const int hh = lane >> 5, l32 = lane & 31;
  const float* kb = w.kbar + ((size_t)h * dm.Nb + j) * 128;
  const float* vs = w.vsum + ((size_t)h * dm.Nb + j) * 128;
  const float* hb = w.hbar + (size_t)h * 128 * 128;
  float ss = 0.f;
  // H_j^T in bf16 for the block-wise first-order variant (row b holds H_j[:, b])
  __bf16* hjt = reinterpret_cast<__bf16*>(w.hjT_lo) + ((size_t)h * dm.Nb + j) * 128 * 128;
  for (int ct = 0; ct < 4; ++ct) {
    const int b = 32 * ct + l32;
    const float vb = vs[b];
    for (int g = 0; g < 4; ++g) {
      bf16x4 hj;
      for (int r = 0; r < 4; ++r) {
        const int x = 4 * g + r;
        const int a = 32 * wave + 8 * g + 4 * hh + r;
        const float h_ab = acc[ct][x] - kb[a] * vb;
        const float hv = h_ab - hb[a * 128 + b];
        ss += hv * hv;
        if constexpr (HJT) hj[r] = (__bf16)h_ab;
        if constexpr (SPEC) spec.E[a][b] = hv;
      }
      if constexpr (HJT) *reinterpret_cast<bf16x4*>(hjt + b * 128 + 32 * wave + 8 * g + 4 * hh) = hj;
    }
  }
  if constexpr (SPEC) {
    __syncthreads();
    const float sn = spectral_norm<128>(spec, tid);
    if (tid == 0) w.M[(size_t)h * dm.Nb + j] = sn;
    return;
  }
  ss = wave_sum(ss);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  if (tid == 0) w.M[(size_t)h * dm.Nb + j] = sqrtf(red[0] + red[1] + red[2] + red[3]);
}

// ---------------------------------------------------------------------------------------------
// fp32 inputs: plain FMA. Each thread owns a P x P patch of the D x D product (P = D / 16).
// ---------------------------------------------------------------------------------------------

template <int D, bool COV, bool SPEC = false>
__global__ __launch_bounds__(256) void stats_f32(Dims dm, Work w, const float* __restrict__ Q,
                                                 const float* __restrict__ K, const float* __restrict__ V) {
  constexpr int P = D / 16;
  constexpr int SUB = 32;  // rows per LDS sub-tile
  __shared__ float Ks[SUB][D + 4];
  __shared__ float Vs[SUB][D + 4];
  __shared__ float red[256 / 64];
  __shared__ SpecLds<SPEC ? D : 1> spec;
  __shared__ float ckb[D], cvs[D];  // centroid and value sum of the current block (pass A)
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int a0 = P * (tid / 16), b0 = P * (tid % 16);
  int j0, j1;
  if (COV) {
    j0 = blockIdx.x;
    j1 = j0 + 1;
  } else {
    j0 = blockIdx.x * dm.chunk;
    j1 = min(dm.Nb, j0 + dm.chunk);
  }
  float acc[P][P];
  for (int x = 0; x < P; ++x)
    for (int y = 0; y < P; ++y) acc[x][y] = 0.f;
  for (int j = j0; j < j1; ++j) {
    const int n = (j == dm.Nb - 1) ? dm.n_last : dm.B;
    const size_t r0 = (size_t)h * dm.L * D + (size_t)j * dm.B * D;
    if (COV)
      for (int x = 0; x < P; ++x)
        for (int y = 0; y < P; ++y) acc[x][y] = 0.f;
    if (!COV) __syncthreads();  // every thread done with the previous block's ckb / cvs
    if (!COV && tid < D) {
      float sq = 0.f, sk = 0.f, sv = 0.f;
      for (int r = 0; r < n; ++r) {
        sq += Q[r0 + (size_t)r * D + tid];
        sk += K[r0 + (size_t)r * D + tid];
        sv += V[r0 + (size_t)r * D + tid];
      }
      const size_t o = ((size_t)h * dm.Nb + j) * D + tid;
      w.qbar[o] = sq * dm.scale / (float)n;
      w.kbar[o] = sk / (float)n;
      w.vsum[o] = sv;
      ckb[tid] = sk / (float)n;
      cvs[tid] = sv;
    }
    for (int s0 = 0; s0 < n; s0 += SUB) {
      __syncthreads();
      for (int e = tid; e < SUB * D; e += 256) {
        const int r = e / D, cc = e % D;
        const bool ok = s0 + r < n;
        Ks[r][cc] = ok ? K[r0 + (size_t)(s0 + r) * D + cc] : 0.f;
        Vs[r][cc] = ok ? V[r0 + (size_t)(s0 + r) * D + cc] : 0.f;
      }
      __syncthreads();
      for (int r = 0; r < SUB; ++r)
        for (int x = 0; x < P; ++x) {
          const float kv = Ks[r][a0 + x];
          for (int y = 0; y < P; ++y) acc[x][y] += kv * Vs[r][b0 + y];
        }
    }
    if (!COV) {  // the chunk partial sums H_j = K_j^T V_j - kbar_j (sum V_j)^T
      for (int x = 0; x < P; ++x)
        for (int y = 0; y < P; ++y) acc[x][y] = fmaf(-ckb[a0 + x], cvs[b0 + y], acc[x][y]);
    }
    if (COV) {
      const float* kb = w.kbar + ((size_t)h * dm.Nb + j) * D;
      const float* vs = w.vsum + ((size_t)h * dm.Nb + j) * D;
      const float* hb = w.hbar + (size_t)h * D * D;
      float ss = 0.f;
      for (int x = 0; x < P; ++x)
        for (int y = 0; y < P; ++y) {
          const float hv = acc[x][y] - kb[a0 + x] * vs[b0 + y] - hb[(a0 + x) * D + b0 + y];
          ss += hv * hv;
          if constexpr (SPEC) spec.E[a0 + x][b0 + y] = hv;
        }
      if constexpr (SPEC) {
        __syncthreads();
        const float sn = spectral_norm<D>(spec, tid);
        if (tid == 0) w.M[(size_t)h * dm.Nb + j] = sn;
        continue;
      }
      ss = wave_sum(ss);
      if ((tid & 63) == 0) red[tid >> 6] = ss;
      __syncthreads();
      if (tid == 0) w.M[(size_t)h * dm.Nb + j] = sqrtf(red[0] + red[1] + red[2] + red[3]);
    }
  }
  if (!COV) {
    float* G = w.G + ((size_t)h * dm.NC + blockIdx.x) * D * D;
    for (int x = 0; x < P; ++x)
      for (int y = 0; y < P; ++y) G[(a0 + x) * D + b0 + y] = acc[x][y];
  }
}

// ---------------------------------------------------------------------------------------------
// Finalize: H-bar = (sum_c G_c) / N_b (the partials already hold sum_{j in c} H_j), and (bf16 path)
// bf16 pooled tokens and H-bar^T. Grid (D * D / 256, H): one H-bar entry per thread; pooled rows
// are spread over the same grid.
// ---------------------------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(256) void stats_finalize(Dims dm, Work w) {
  const int h = blockIdx.y, x = blockIdx.x, tid = threadIdx.x;
  const int e = x * 256 + tid;  // entry a * D + b
  const int a = e / D, b = e % D;
  const float* G = w.G + (size_t)h * dm.NC * D * D + e;
  float g0 = 0.f, g1 = 0.f, g2 = 0.f, g3 = 0.f;
  int c = 0;
  for (; c + 4 <= dm.NC; c += 4) {
    g0 += G[(size_t)c * D * D];
    g1 += G[(size_t)(c + 1) * D * D];
    g2 += G[(size_t)(c + 2) * D * D];
    g3 += G[(size_t)(c + 3) * D * D];
  }
  for (; c < dm.NC; ++c) g0 += G[(size_t)c * D * D];
  const float v = ((g0 + g1) + (g2 + g3)) / (float)dm.Nb;
  w.hbar[(size_t)h * D * D + e] = v;
  if (dm.dtype == 0) {
    reinterpret_cast<__bf16*>(w.hbarT_lo)[(size_t)h * D * D + b * D + a] = (__bf16)v;
    const float* kb = w.kbar + (size_t)h * dm.Nb * D;
    const float* vs = w.vsum + (size_t)h * dm.Nb * D;
    __bf16* kl = reinterpret_cast<__bf16*>(w.kbar_lo) + (size_t)h * dm.Nbp * D;
    __bf16* vl = reinterpret_cast<__bf16*>(w.vbar_lo) + (size_t)h * dm.Nbp * D;
    const int per = 256 / D;  // pooled rows per workgroup pass
    for (int j = x * per + tid / D; j < dm.Nbp; j += gridDim.x * per) {
      const int cc = tid % D;
      float kv = 0.f, vv = 0.f;
      if (j < dm.Nb) {
        const float n = (j == dm.Nb - 1) ? (float)dm.n_last : (float)dm.B;
        kv = kb[(size_t)j * D + cc];
        vv = vs[(size_t)j * D + cc] / n;
      }
      kl[(size_t)j * D + cc] = (__bf16)kv;
      vl[(size_t)j * D + cc] = (__bf16)vv;
    }
  }
}

}  // namespace

hipError_t launch_stats_pass_bf16(const Dims& dm, const Work& w, const void* Q, const void* K, const void* V,
                                  hipStream_t s) {
  dim3 grid(dm.NC, dm.H);
  auto q = static_cast<const __bf16*>(Q);
  auto k = static_cast<const __bf16*>(K);
  auto v = static_cast<const __bf16*>(V);
  if (dm.B == 128)
    hipLaunchKernelGGL(stats_pass_bf16<128>, grid, dim3(256), 0, s, dm, w, q, k, v);
  else
    hipLaunchKernelGGL(stats_pass_bf16<64>, grid, dim3(256), 0, s, dm, w, q, k, v);
  return hipGetLastError();
}

hipError_t launch_stats_cov_bf16(const Dims& dm, const Work& w, const void* K, const void* V, hipStream_t s) {
  dim3 grid(dm.Nb, dm.H);
  auto k = static_cast<const __bf16*>(K);
  auto v = static_cast<const __bf16*>(V);
#define PISA_COV(BLK, SPEC, HJT) \
  hipLaunchKernelGGL((stats_cov_bf16<BLK, SPEC, HJT>), grid, dim3(256), 0, s, dm, w, k, v)
  const bool hjt = block_first_order(dm);
  if (dm.B == 128) {
    if (dm.spectral) {
      if (hjt) PISA_COV(128, true, true); else PISA_COV(128, true, false);
    } else {
      if (hjt) PISA_COV(128, false, true); else PISA_COV(128, false, false);
    }
  } else {
    if (dm.spectral) {
      if (hjt) PISA_COV(64, true, true); else PISA_COV(64, true, false);
    } else {
      if (hjt) PISA_COV(64, false, true); else PISA_COV(64, false, false);
    }
  }
#undef PISA_COV
  return hipGetLastError();
}

hipError_t launch_stats_pass_f32(const Dims& dm, const Work& w, const void* Q, const void* K, const void* V,
                                 hipStream_t s) {
  dim3 grid(dm.NC, dm.H);
  auto q = static_cast<const float*>(Q);
  auto k = static_cast<const float*>(K);
  auto v = static_cast<const float*>(V);
  if (dm.d == 128)
    hipLaunchKernelGGL((stats_f32<128, false>), grid, dim3(256), 0, s, dm, w, q, k, v);
  else
    hipLaunchKernelGGL((stats_f32<64, false>), grid, dim3(256), 0, s, dm, w, q, k, v);
  return hipGetLastError();
}

hipError_t launch_stats_cov_f32(const Dims& dm, const Work& w, const void* K, const void* V, hipStream_t s) {
  dim3 grid(dm.Nb, dm.H);
  auto k = static_cast<const float*>(K);
  auto v = static_cast<const float*>(V);
  if (dm.spectral) {
    if (dm.d == 128)
      hipLaunchKernelGGL((stats_f32<128, true, true>), grid, dim3(256), 0, s, dm, w, nullptr, k, v);
    else
      hipLaunchKernelGGL((stats_f32<64, true, true>), grid, dim3(256), 0, s, dm, w, nullptr, k, v);
  } else {
    if (dm.d == 128)
      hipLaunchKernelGGL((stats_f32<128, true>), grid, dim3(256), 0, s, dm, w, nullptr, k, v);
    else
      hipLaunchKernelGGL((stats_f32<64, true>), grid, dim3(256), 0, s, dm, w, nullptr, k, v);
  }
  return hipGetLastError();
}

hipError_t launch_stats_finalize(const Dims& dm, const Work& w, hipStream_t s) {
  dim3 grid(dm.d * dm.d / 256, dm.H);
  if (dm.d == 128)
    hipLaunchKernelGGL(stats_finalize<128>, grid, dim3(256), 0, s, dm, w);
  else
    hipLaunchKernelGGL(stats_finalize<64>, grid, dim3(256), 0, s, dm, w);
  return hipGetLastError();
}

}  // namespace pisa
