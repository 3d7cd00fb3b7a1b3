// Block statistics for PISA (the precompute step of the fused kernel described on the
// gist.science summary of the PISA paper, section 2 "Hardware implementation"; the statistics
// themselves follow section 2 "Core algorithm" - centroid and value sum of every block - and
// "Covariance-aware routing" - the block first-order matrices H_j, their mean H-bar and
// M_j = ||H_j - H-bar||).
//
// Pass A: column sums of Q, K, V per block (pooled scaled query, key centroid, value sum) and
// partial sums of the block first-order matrices H_j = K_j^T V_j - kbar_j (sum V_j)^T
// (= sum_n (k_n - kbar_j)^T v_n). fp32 inputs: one workgroup per chunk of up to 16 consecutive
// blocks of a head. bf16 inputs: one workgroup per range of consecutive (head, block) pairs, the
// ranges of equal length over all heads (one round of workgroups on the chip, one partial per head
// a range meets); the Q column sums are a kernel of their own (stats_qbar_bf16), so that pass A's
// loop moves only K and V.
// Finalize (per head): H-bar = (sum of the partials) / N_b; bf16 copies of the pooled tokens and
// of H-bar^T for the attention kernel. Covariance pass (bf16 Frobenius norm: the statistics pass's
// ranges; fp32, the spectral norm and the H_j^T variant: one workgroup per block): H_j again, then
// M_j = ||H_j - H-bar|| (and H_j^T in bf16 for the block-wise first-order variant).
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

// The same product, plus the column sums on the matrix unit: ksum += K^T 1 (the K^T operand
// against a ones operand) and vsum += 1^T V for the wave's own 32 columns, over the BLK rows of the
// tiles (acc, ksum and vsum accumulate; the caller clears them). Products with 1.0 are exact and
// the sums accumulate in fp32. Rows past the block end are zero in the tiles.
// Lane l holds: ksum[x] = column sum of K for d = 32 wave + 8 (x >> 2) + 4 (l >> 5) + (x & 3);
// vsum[0] = column sum of V for column 32 wave + (l & 31).
template <int BLK>
__device__ __forceinline__ void ktv_mfma_sums(const char* Ks, const char* Vs, f32x16 acc[4], f32x16& ksum,
                                              f32x16& vsum, int wave, int lane) {
  const uint32_t hh = lane >> 5, g16 = (lane >> 4) & 1, l16 = lane & 15;
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
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

// Q column sums, bf16 (the pooled scaled query of every block): one workgroup per block, each thread
// summing 16-byte pieces of its rows in registers, then across the 16-lane row groups and across
// waves. A plain streaming reduction with many small workgroups per CU.
template <int BLK>
__global__ __launch_bounds__(256) void stats_qbar_bf16(Dims dm, Work w, const __bf16* __restrict__ Q) {
  __shared__ float red[4][128];
  constexpr int QR = BLK / 16;  // 16-byte pieces per thread
  const int h = blockIdx.y, j = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int p = tid & 15, rg = tid >> 4;  // column chunk (8 columns) and row group
  const int n = (j == dm.Nb - 1) ? dm.n_last : dm.B;
  const size_t r0 = (size_t)h * dm.L * 128 + (size_t)j * dm.B * 128;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + r0, n * 256);
  u32x4 qa[QR];
#pragma unroll
  for (int e = 0; e < QR; ++e)  // read once: non-temporal (cache policy bit 1)
    qa[e] = __builtin_amdgcn_raw_buffer_load_b128(rq, (rg + 16 * e) * 256 + p * 16, 0, 2);
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
  __syncthreads();
  if (tid < 128)
    w.qbar[((size_t)h * dm.Nb + j) * 128 + tid] =
        (red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid]) * dm.scale * (1.0f / (float)n);
}

// The statistics pass and the covariance pass (bf16) stream a block's K and V tiles through LDS
// in two halves of BLK/2 rows (the half-block ring): half h of the next block is copied into half
// h's slots as soon as every wave has read half h of the current block, so one half is in flight
// while the other is multiplied, and a CU (two workgroups, 64 KB of slots each) always has copies
// outstanding. A half starts at a row that is a multiple of 16, so the tiles' swizzle is the same
// as for the whole block; rows of a half past the block end are written as zeros (each 16-row
// chunk's buffer resource ends where the block's rows end).
//
// Each pass reads every K and V byte once: the copies carry the non-temporal hint, so that the two
// streams do not displace other lines (the passes' own output rows among them) from L2.
//
// The copies are issued from assembly (copy_tile_chunks), out of sight of the compiler's
// wait-count insertion, which cannot tell copies into one slot from reads of the other and would
// make every read wait for the latest copy. The loops issue no other global loads (the covariance
// pass's H-bar rows, loaded when a range enters a head, are followed by a full wait), so the waits
// below (for all but the copies of the half issued after the one needed) are the only ones.
template <int BLK>
__device__ __forceinline__ void kv_half_copy(const __bf16* K, const __bf16* V, size_t r0, int n, int half,
                                             uint32_t kslot, uint32_t vslot, uint32_t v0, int wave) {
  constexpr int HR = BLK / 2;
  const uint32_t bytes = 256u * (uint32_t)__builtin_amdgcn_readfirstlane(max(0, min(HR, n - HR * half)));
  const __bf16* kb = K + r0 + (size_t)HR * half * 128;
  const __bf16* vb = V + r0 + (size_t)HR * half * 128;
  if constexpr (HR % 64 == 0) {  // every wave copies a chunk of K and one of V
    copy_tile_chunks<HR, 4, true, true>(kb, bytes, kslot, v0, wave);
    copy_tile_chunks<HR, 4, true, true>(vb, bytes, vslot, v0, wave);
  } else {  // 32-row halves: waves 0-1 copy K's two chunks, waves 2-3 V's
    static_assert(HR == 32, "half-block rows");
    if (wave < 2) copy_tile_chunks<HR, 2, true, true>(kb, bytes, kslot, v0, wave);
    else copy_tile_chunks<HR, 2, true, true>(vb, bytes, vslot, v0, wave - 2);
  }
}

// Copy instructions each thread issues per half (4 per 16-row chunk).
template <int BLK>
constexpr int kv_half_vmem() { return (BLK / 2) % 64 == 0 ? 2 * (BLK / 2) / 16 : 4; }

// Workgroup barrier that orders LDS accesses only: each wave's LDS reads and writes have completed
// (lgkmcnt(0)) before any wave passes. Unlike __syncthreads() it does not wait for the wave's
// outstanding copies and stores, so the ring's next half stays in flight across it. The "memory"
// clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __asm__ __volatile__("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt vmcnt(N), expcnt and lgkmcnt at their maxima (N < 16). Vector-memory loads complete
// in issue order: once at most N operations are outstanding, every load issued before the N most
// recent operations has landed.
template <int N>
__device__ __forceinline__ void wait_vmem_but() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
  __asm__ __volatile__("" ::: "memory");
}

// Pass A, bf16: column sums of K and V and K^T V (matrix unit, from LDS) over the workgroup's range
// of (head, block) pairs, through the half-block ring, which runs on across head boundaries. For each
// head the range meets, the partial is corrected by the centroids block by block,
// G = sum_j (K_j^T V_j - kbar_j (sum V_j)^T) = sum_j H_j over the range's blocks of that head, and
// written with the centroids' partial sum to the head's slot when the range leaves the head. The Q
// column sums are stats_qbar_bf16's.
template <int BLK>
__global__ __launch_bounds__(256, 2) void stats_pass_bf16(Dims dm, Work w, const __bf16* __restrict__ K,
                                                          const __bf16* __restrict__ V) {
  __shared__ __attribute__((aligned(1024))) char Ks0[BLK * 128];  // half-block slots
  __shared__ __attribute__((aligned(1024))) char Ks1[BLK * 128];
  __shared__ __attribute__((aligned(1024))) char Vs0[BLK * 128];
  __shared__ __attribute__((aligned(1024))) char Vs1[BLK * 128];
  // centroids and value sums of a group of up to kStage consecutive blocks, stored together
  constexpr int kStage = 8;
  __shared__ __attribute__((aligned(16))) float stk[kStage * 128];
  __shared__ __attribute__((aligned(16))) float stv[kStage * 128];
  constexpr int HR = BLK / 2;
  constexpr int NV = kv_half_vmem<BLK>();
  const int wg = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g0 = stat_range_begin(dm, wg), g1 = stat_range_begin(dm, wg + 1);
  const uint32_t hh = lane >> 5, l32 = lane & 31;
  const uint32_t v0 = chunk_lane<true>(lane);
  const uint32_t k0 = lds_addr(Ks0), k1 = lds_addr(Ks1), s0 = lds_addr(Vs0), s1 = lds_addr(Vs1);
  f32x16 acc[4];
  for (int ct = 0; ct < 4; ++ct) acc[ct] = f32x16{};
  // the head's sum of block centroids over the range so far; every lane holds the rows of its
  // accumulator entries (a = 32 wave + 8 (x >> 2) + 4 hh + (x & 3)), lanes l32 = 0 write them
  float kc[16];
#pragma unroll
  for (int x = 0; x < 16; ++x) kc[x] = 0.f;

  auto rows_of = [&](int j) { return (j == dm.Nb - 1) ? dm.n_last : dm.B; };
  auto issue = [&](int g, int half) __attribute__((always_inline)) {
    const int h = g / dm.Nb, j = g - h * dm.Nb;
    kv_half_copy<BLK>(K, V, (size_t)h * dm.L * 128 + (size_t)j * dm.B * 128, rows_of(j), half, half ? k1 : k0,
                      half ? s1 : s0, v0, wave);
  };
  // A store issued inside the ring counts against the copies' wait that follows it: a group's
  // outputs are therefore stored at once, after the first barrier of the block that follows the
  // group (or after the loop), one 16-byte piece per thread and array: pairs pg .. pg + cnt - 1 are
  // consecutive rows of kbar and vsum.
  auto store_group = [&](int pg, int cnt) __attribute__((always_inline)) {
    if (4 * tid < cnt * 128) {
      *reinterpret_cast<float4*>(w.kbar + (size_t)pg * 128 + 4 * tid) = *reinterpret_cast<const float4*>(stk + 4 * tid);
      *reinterpret_cast<float4*>(w.vsum + (size_t)pg * 128 + 4 * tid) = *reinterpret_cast<const float4*>(stv + 4 * tid);
    }
  };
  if (g0 < g1) {
    issue(g0, 0);
    issue(g0, 1);
  }
  for (int g = g0; g < g1; ++g) {
    const int h = g / dm.Nb, j = g - h * dm.Nb;
    const int n = rows_of(j);
    const bool more = g + 1 < g1;
    const int sl = (g - g0) % kStage;  // the block's row in the group's staging arrays
    f32x16 ksum = f32x16{}, vsum = f32x16{};
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      // half (g, half) landed; the half issued after it, if any, stays in flight. Loads complete
      // in issue order, so stores issued between the copies do not weaken the count.
      if (half == 0 || more) wait_vmem_but<NV>(); else wait_vmem();
      lds_barrier();
      if (half == 0 && g > g0 && sl == 0) store_group(g - kStage, kStage);
      ktv_mfma_sums<HR>(half ? Ks1 : Ks0, half ? Vs1 : Vs0, acc, ksum, vsum, wave, lane);
      lds_barrier();  // every wave done with this half's slots
      if (more) issue(g + 1, half);
    }
    const float inv = 1.0f / (float)n;
    // lane l's ksum[x] is the column sum of K for row a = 32 wave + 8 (x >> 2) + 4 hh + (x & 3) of
    // the product, the same row as acc[.][x]
    float pk[16];
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      pk[x] = ksum[x] * inv;
      kc[x] += pk[x];
    }
    float* rk = stk + sl * 128;
    float* rv = stv + sl * 128;
    if (l32 == 0) {  // rows 32 wave + 8 q + 4 hh + (0..3): four consecutive floats per q
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(rk + 32 * wave + 8 * q + 4 * hh) =
            make_float4(pk[4 * q], pk[4 * q + 1], pk[4 * q + 2], pk[4 * q + 3]);
    }
    if (lane < 32) rv[32 * wave + lane] = vsum[0];
    lds_barrier();  // the block's row complete (the row is next written kStage blocks on)
    // acc[ct][x] -= kbar_j[a] vsum_j[b], b = 32 ct + l32
    float vb[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) vb[ct] = rv[32 * ct + l32];
#pragma unroll
    for (int x = 0; x < 16; ++x) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) acc[ct][x] = fmaf(-pk[x], vb[ct], acc[ct][x]);
    }
    if (!more || j == dm.Nb - 1) {  // the range leaves head h: its partials go to slot wg + h
      const size_t slot = (size_t)wg + h;
      float* G = w.G + slot * 128 * 128;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const int a = 32 * wave + 8 * (x >> 2) + 4 * hh + (x & 3);
          G[a * 128 + 32 * ct + l32] = acc[ct][x];
          acc[ct][x] = 0.f;
        }
      if (l32 == 0) {
        float* kp = w.kpart + slot * 128;
#pragma unroll
        for (int x = 0; x < 16; ++x) kp[32 * wave + 8 * (x >> 2) + 4 * hh + (x & 3)] = kc[x];
      }
#pragma unroll
      for (int x = 0; x < 16; ++x) kc[x] = 0.f;
    }
  }
  if (g0 < g1) {
    const int cnt = (g1 - 1 - g0) % kStage + 1;
    store_group(g1 - cnt, cnt);
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

// Covariance pass, Frobenius M_j (the default): one workgroup per range of (head, block) pairs, the
// statistics pass's ranges, through the same half-block ring, with the lane's 64 entries of H-bar
// held in registers (loaded again when the range enters another head). The block's centroid and value sums are formed again on the matrix unit beside K^T V
// (the same instructions in the same order as the statistics pass, so the same values) rather
// than read back: the loop then issues no global loads besides the copies and the H-bar rows.
template <int BLK>
__global__ __launch_bounds__(256, 2) void stats_cov_chunk_bf16(Dims dm, Work w, const __bf16* __restrict__ K,
                                                               const __bf16* __restrict__ V) {
  __shared__ __attribute__((aligned(1024))) char Ks0[BLK * 128];  // half-block slots
  __shared__ __attribute__((aligned(1024))) char Ks1[BLK * 128];
  __shared__ __attribute__((aligned(1024))) char Vs0[BLK * 128];
  __shared__ __attribute__((aligned(1024))) char Vs1[BLK * 128];
  __shared__ float svs[2][128];  // value sums of the block (alternating buffers)
  __shared__ float red[2][4];
  // M of a group of up to kStage consecutive blocks, stored together: a store issued inside the
  // ring counts against the copies' wait that follows it
  constexpr int kStage = 8;
  __shared__ float sM[kStage];
  constexpr int HR = BLK / 2;
  constexpr int NV = kv_half_vmem<BLK>();
  const int wg = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, l32 = lane & 31;
  const int g0 = stat_range_begin(dm, wg), g1 = stat_range_begin(dm, wg + 1);
  const uint32_t v0 = chunk_lane<true>(lane);
  const uint32_t k0 = lds_addr(Ks0), k1 = lds_addr(Ks1), s0 = lds_addr(Vs0), s1 = lds_addr(Vs1);
  auto rows_of = [&](int j) { return (j == dm.Nb - 1) ? dm.n_last : dm.B; };
  auto issue = [&](int g, int half) __attribute__((always_inline)) {
    const int h = g / dm.Nb, j = g - h * dm.Nb;
    kv_half_copy<BLK>(K, V, (size_t)h * dm.L * 128 + (size_t)j * dm.B * 128, rows_of(j), half, half ? k1 : k0,
                      half ? s1 : s0, v0, wave);
  };
  auto m_of = [&](int t) { return sqrtf(red[t & 1][0] + red[t & 1][1] + red[t & 1][2] + red[t & 1][3]); };
  if (g0 < g1) {
    issue(g0, 0);
    issue(g0, 1);
  }
  float hbr[4][16];  // H-bar[a][b] for the lane's accumulator entries (a, b as in acc[ct][x])
  int hcur = -1;
  for (int t = 0; t < g1 - g0; ++t) {
    const int g = g0 + t;
    const int h = g / dm.Nb, j = g - h * dm.Nb;
    const bool more = g + 1 < g1;
    const bool fresh = h != hcur;
    if (fresh) {
      // through a buffer resource: one lane offset, the entry's offset an immediate or a scalar
      const __amdgpu_buffer_rsrc_t rh = make_rsrc(w.hbar + (size_t)h * 128 * 128, 128 * 128 * 4);
      const uint32_t lo = 4u * ((32 * wave + 4 * hh) * 128 + l32);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int x = 0; x < 16; ++x)
          hbr[ct][x] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
              rh, lo, 4 * ((8 * (x >> 2) + (x & 3)) * 128 + 32 * ct), 0));
      // wait for everything (the copies in flight too): the rows are then complete, and the
      // compiler, which does not count the copies, knows it and inserts no wait of its own later
      wait_vmem();
      hcur = h;
    }
    f32x16 acc[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[ct] = f32x16{};
    f32x16 ksum = f32x16{}, vsum = f32x16{};
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      // half (g, half) landed; the half issued after it, if any, stays in flight (the stores
      // issued since are younger still)
      if (half == 0 || more) wait_vmem_but<NV>(); else wait_vmem();
      lds_barrier();
      if (half == 0 && t > 0) {  // M of the previous block (pair g - 1)
        if (tid == 0) sM[(t - 1) % kStage] = m_of(t - 1);
        // a complete group, pairs g - kStage .. g - 1, by wave 0 (which wrote sM; its LDS accesses
        // are done in order)
        if ((t - 1) % kStage == kStage - 1 && tid < kStage) w.M[g - kStage + tid] = sM[tid];
      }
      ktv_mfma_sums<HR>(half ? Ks1 : Ks0, half ? Vs1 : Vs0, acc, ksum, vsum, wave, lane);
      lds_barrier();  // every wave done with this half's slots
      if (more) issue(g + 1, half);
    }
    const float inv = 1.0f / (float)rows_of(j);
    if (lane < 32) svs[t & 1][32 * wave + lane] = vsum[0];
    lds_barrier();  // svs[t & 1] complete; it is next written two blocks on, after several barriers
    float ss = 0.f;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const float vb = svs[t & 1][32 * ct + l32];
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const float hv = fmaf(-(ksum[x] * inv), vb, acc[ct][x]) - hbr[ct][x];
        ss = fmaf(hv, hv, ss);
      }
    }
    ss = wave_sum(ss);
    if (lane == 0) red[t & 1][wave] = ss;  // read after the next block's first barrier
  }
  if (g0 < g1) {  // the last block's M, then the last group (pairs g1 - cnt .. g1 - 1)
    lds_barrier();
    const int n = g1 - g0, cnt = (n - 1) % kStage + 1;
    if (tid == 0) sM[(n - 1) % kStage] = m_of(n - 1);
    if (tid < cnt) w.M[g1 - cnt + tid] = sM[tid];
  }
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
#pragma unroll 8
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
      {  // 16-byte loads, all of the thread's in flight before the first store
        constexpr int kPer = SUB * D / 4 / 256;
        f32x4 kv4[kPer], vv4[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
          const int e = 4 * (tid + 256 * u), r = e / D, cc = e % D;
          const bool ok = s0 + r < n;
          const size_t g = r0 + (size_t)(s0 + r) * D + cc;
          kv4[u] = ok ? *reinterpret_cast<const f32x4*>(K + g) : f32x4{0.f, 0.f, 0.f, 0.f};
          vv4[u] = ok ? *reinterpret_cast<const f32x4*>(V + g) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
          const int e = 4 * (tid + 256 * u), r = e / D, cc = e % D;
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            Ks[r][cc + x] = kv4[u][x];
            Vs[r][cc + x] = vv4[u][x];
          }
        }
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
// Finalize: H-bar = (sum of the head's partials G) / N_b (each partial already holds the sum of H_j
// over its blocks, summed here in slot order), and (bf16 path) bf16 pooled tokens and H-bar^T. Grid (D * D / 256, H): one H-bar entry per thread; pooled rows
// are spread over the same grid.
// ---------------------------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(256) void stats_finalize(Dims dm, Work w) {
  const int h = blockIdx.y, x = blockIdx.x, tid = threadIdx.x;
  const int e = x * 256 + tid;  // entry a * D + b
  const int a = e / D, b = e % D;
  // the head's partial slots: fp32 path h NC .. h NC + NC - 1, bf16 path those of the ranges that
  // meet head h
  const bool cen = dm.dtype == 0;
  const int p0 = cen ? stat_owner(dm, h * dm.Nb) + h : h * dm.NC;
  const int np = cen ? stat_owner(dm, h * dm.Nb + dm.Nb - 1) + h + 1 - p0 : dm.NC;
  const float* G = w.G + (size_t)p0 * D * D + e;
  // bf16 path: the partial sums of the block centroids (column tid % D) are added in the same
  // loop, so their loads are in flight together with the partials of H-bar
  const float* kp = cen ? w.kpart + (size_t)p0 * D + (tid % D) : G;
  float g0 = 0.f, g1 = 0.f, g2 = 0.f, g3 = 0.f, k0 = 0.f, k1 = 0.f, k2 = 0.f, k3 = 0.f;
  int c = 0;
  for (; c + 4 <= np; c += 4) {
    g0 += G[(size_t)c * D * D];
    g1 += G[(size_t)(c + 1) * D * D];
    g2 += G[(size_t)(c + 2) * D * D];
    g3 += G[(size_t)(c + 3) * D * D];
    if (cen) {
      k0 += kp[(size_t)c * D];
      k1 += kp[(size_t)(c + 1) * D];
      k2 += kp[(size_t)(c + 2) * D];
      k3 += kp[(size_t)(c + 3) * D];
    }
  }
  for (; c < np; ++c) {
    g0 += G[(size_t)c * D * D];
    if (cen) k0 += kp[(size_t)c * D];
  }
  const float v = ((g0 + g1) + (g2 + g3)) / (float)dm.Nb;
  w.hbar[(size_t)h * D * D + e] = v;
  if (dm.dtype == 0) {
    reinterpret_cast<__bf16*>(w.hbarT_lo)[(size_t)h * D * D + b * D + a] = (__bf16)v;
    const float* kb = w.kbar + (size_t)h * dm.Nb * D;
    const float* vs = w.vsum + (size_t)h * dm.Nb * D;
    __bf16* kl = reinterpret_cast<__bf16*>(w.kbar_lo) + (size_t)h * dm.Nbp * D;
    __bf16* vl = reinterpret_cast<__bf16*>(w.vbar_lo) + (size_t)h * dm.Nbp * D;
    const int per = 256 / D;  // pooled rows per workgroup pass
    const int cc = tid % D;
    // key centre c = mean of the block centroids (chunk sums added in a fixed order). The bf16
    // pooled centroids are stored relative to it: keys that share a large common component then
    // keep their differences to bf16 precision, and the attention kernel adds q.c back in fp32.
    const float kcen = ((k0 + k1) + (k2 + k3)) / (float)dm.Nb;
    if (x == 0 && tid < D) w.kc[(size_t)h * D + cc] = kcen;
    for (int j = x * per + tid / D; j < dm.Nbp; j += gridDim.x * per) {
      float kv = 0.f, vv = 0.f;
      if (j < dm.Nb) {
        const float n = (j == dm.Nb - 1) ? (float)dm.n_last : (float)dm.B;
        kv = kb[(size_t)j * D + cc] - kcen;
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
  dim3 grid(dm.SW), qgrid(dm.Nb, dm.H);
  auto q = static_cast<const __bf16*>(Q);
  auto k = static_cast<const __bf16*>(K);
  auto v = static_cast<const __bf16*>(V);
  if (dm.B == 128) {
    hipLaunchKernelGGL(stats_qbar_bf16<128>, qgrid, dim3(256), 0, s, dm, w, q);
    hipLaunchKernelGGL(stats_pass_bf16<128>, grid, dim3(256), 0, s, dm, w, k, v);
  } else {
    hipLaunchKernelGGL(stats_qbar_bf16<64>, qgrid, dim3(256), 0, s, dm, w, q);
    hipLaunchKernelGGL(stats_pass_bf16<64>, grid, dim3(256), 0, s, dm, w, k, v);
  }
  return hipGetLastError();
}

hipError_t launch_stats_cov_bf16(const Dims& dm, const Work& w, const void* K, const void* V, hipStream_t s) {
  dim3 grid(dm.Nb, dm.H);
  auto k = static_cast<const __bf16*>(K);
  auto v = static_cast<const __bf16*>(V);
#define PISA_COV(BLK, SPEC, HJT) \
  hipLaunchKernelGGL((stats_cov_bf16<BLK, SPEC, HJT>), grid, dim3(256), 0, s, dm, w, k, v)
  const bool hjt = block_first_order(dm);
  if (!dm.spectral && !hjt) {
    dim3 cgrid(dm.SW);
    if (dm.B == 128)
      hipLaunchKernelGGL(stats_cov_chunk_bf16<128>, cgrid, dim3(256), 0, s, dm, w, k, v);
    else
      hipLaunchKernelGGL(stats_cov_chunk_bf16<64>, cgrid, dim3(256), 0, s, dm, w, k, v);
    return hipGetLastError();
  }
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
