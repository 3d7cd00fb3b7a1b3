// Fused piecewise attention, bf16 inputs, d = 128 (gist.science summary of the PISA paper,
// section 2 "Core algorithm" for what is computed and "Hardware implementation" for the phase
// structure: exact blocks, then aggregated block vectors at zeroth order, then the global
// first-order correction, all inside one online softmax).
//
// One workgroup per (head, query block), BLK/32 waves, wave w owning query rows 32w..32w+31.
// Everything is computed transposed so that every per-query quantity lives in the lane that owns
// the query (lane % 32):
//   S^T = K_tile Q^T      A = K rows from LDS (16 B reads), B = Q^T held in registers
//   O^T += V^T P^T        A = V^T via ds_read_b64_tr_b16 from the row-major V tile,
//                         B = P^T straight from the S^T accumulators (converted to bf16)
//   T^T = H-bar^T Q^T     phase 3, same routine as S^T with H-bar^T as the tile
// Lanes l and l^32 hold the two halves of each query's keys (and of its output columns); the row
// max is exchanged between them once per tile, the row sums at the end.
//
// Phase 1: for j in S_i (ascending), K_j and V_j tiles are copied global -> LDS directly
// (buffer loads with the range cut at the block's n_j rows, so ragged rows read as zero) and
// processed flash-style with scores in the log2 domain (scale * log2 e folded into one FMA).
// Phase 2: pooled tokens (kbar_j, vbar_j) in tiles of BLK, with additive bias log2 n_j, masked to
// j in U_i (selection bit mask in LDS) and j < N_b; beta += p / n_j.
// Phase 3: O += (beta * scale) (q H-bar).
// Epilogue: out = O / l, rounded to bf16, transposed through LDS for 16-byte row stores.
#include "dev_common.h"
#include "pisa_internal.h"

namespace pisa {
namespace {

constexpr int kMaskWords = (8192 + 128) / 32;  // N_b <= 8192, rounded up to a tile

// S^T for NT key subtiles of 32 rows: S[t] += Tile[32t + l32][:] . Q^T[:][query]
template <int NT>
__device__ __forceinline__ void qk_tile(const char* tile, const bf16x8 qreg[8], f32x16 S[NT], uint32_t l32,
                                        uint32_t hh) {
#pragma unroll
  for (int t = 0; t < NT; ++t) S[t] = f32x16{};
#pragma unroll
  for (int s = 0; s < 8; ++s)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(row_addr(tile, 32 * t + l32, 2 * s + hh));
      S[t] = mfma32(a, qreg[s], S[t]);
    }
}

// O^T[dt] += V^T P^T over NT key subtiles.
template <int NT>
__device__ __forceinline__ void pv_tile(const char* Vs, const bf16x8 P[NT][2], f32x16 O[4], uint32_t hh,
                                        uint32_t g16, uint32_t l16) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint32_t klo = 32 * t + 16 * u + 4 * hh;
        const bf16x8 a = tr_operand(Vs, klo, klo + 8, 32 * dt + 16 * g16, l16);
        O[dt] = mfma32(a, P[t][u], O[dt]);
      }
}

// Workgroup id -> logical work item, so that each of the 8 XCDs (which receive workgroup ids
// round-robin) walks a contiguous range of (head, query block) items.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int per = n / 8, rem = n % 8;
  const int x = bid % 8, q = bid / 8;
  return x * per + min(x, rem) + q;
}

template <int BLK>
__global__ __launch_bounds__(BLK * 2, 2) void attend_bf16(Dims dm, Work w, const __bf16* __restrict__ Q,
                                                          const __bf16* __restrict__ K,
                                                          const __bf16* __restrict__ V,
                                                          __bf16* __restrict__ out) {
  constexpr int NW = BLK / 32;  // waves
  constexpr int NT = BLK / 32;  // 32-key subtiles per tile
  __shared__ __attribute__((aligned(1024))) char smem[2 * BLK * 256 < 128 * 256 ? 128 * 256 : 2 * BLK * 256];
  __shared__ uint32_t selm[kMaskWords];
  char* Ks = smem;
  char* Vs = smem + BLK * 256;

  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int h = item / dm.Nb, i = item % dm.Nb;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint32_t hh = lane >> 5, l32 = lane & 31, g16 = (lane >> 4) & 1, l16 = lane & 15;
  const int Nb = dm.Nb, B = dm.B, kk = dm.k;
  const int n_i = (i == Nb - 1) ? dm.n_last : B;
  const size_t head = (size_t)h * dm.L * 128;

  // Q^T operand: query row 32*wave + l32 of the block, d = 16 s + 8 hh .. +7
  bf16x8 qreg[8];
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + head + (size_t)i * B * 128, n_i * 256);
    const uint32_t row = 32 * wave + l32;
#pragma unroll
    for (int s = 0; s < 8; ++s) qreg[s] = __builtin_bit_cast(bf16x8, buf_load16(rq, row * 256 + (16 * s + 8 * hh) * 2));
  }

  const int nmask = (dm.Nbp + 31) / 32;
  for (int t = tid; t < nmask; t += BLK * 2) selm[t] = 0u;
  __syncthreads();
  const int32_t* sel = w.idx + ((size_t)h * Nb + i) * kk;
  for (int t = tid; t < kk; t += BLK * 2) {
    const int j = sel[t];
    atomicOr(&selm[j >> 5], 1u << (j & 31));
  }

  const float cs = dm.scale * kLog2e;
  float m = -INFINITY, lsum = 0.f, beta = 0.f;
  f32x16 O[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) O[dt] = f32x16{};
  f32x16 S[NT];
  bf16x8 P[NT][2];

  // ---- phase 1: exact blocks --------------------------------------------------------------
  for (int it = 0; it < kk; ++it) {
    const int j = __builtin_amdgcn_readfirstlane(sel[it]);
    const int n_j = (j == Nb - 1) ? dm.n_last : B;
    const size_t r0 = head + (size_t)j * B * 128;
    tile_to_lds<false>(make_rsrc(K + r0, n_j * 256), 256, Ks, BLK, wave, NW, lane);
    tile_to_lds<true>(make_rsrc(V + r0, n_j * 256), 256, Vs, BLK, wave, NW, lane);
    wait_vmem();
    __syncthreads();
    qk_tile<NT>(Ks, qreg, S, l32, hh);
    if (n_j < BLK) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const int key = 32 * t + 8 * (x >> 2) + 4 * hh + (x & 3);
          if (key >= n_j) S[t][x] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int x = 0; x < 16; ++x) mx = fmaxf(mx, S[t][x]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx * cs);
    const float alpha = m == m_new ? 1.0f : __builtin_amdgcn_exp2f(m - m_new);
    m = m_new;
    lsum *= alpha;
    beta *= alpha;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) O[dt] *= alpha;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(fmaf(S[t][8 * u + e], cs, -m));
          lsum += p;
          P[t][u][e] = (__bf16)p;
        }
    pv_tile<NT>(Vs, P, O, hh, g16, l16);
    __syncthreads();
  }

  const bool do_tail = kk < Nb && (dm.phases & 2);
  // ---- phase 2: pooled tokens of the unselected blocks, zeroth order ---------------------------
  if (do_tail) {
    const float lgB = __log2f((float)B), lgLast = __log2f((float)dm.n_last);
    const float invB = 1.0f / (float)B, invLast = 1.0f / (float)dm.n_last;
    const __bf16* kl = reinterpret_cast<const __bf16*>(w.kbar_lo) + (size_t)h * dm.Nbp * 128;
    const __bf16* vl = reinterpret_cast<const __bf16*>(w.vbar_lo) + (size_t)h * dm.Nbp * 128;
    for (int c = 0; c < dm.Nbp / BLK; ++c) {
      const size_t r0 = (size_t)c * BLK * 128;
      tile_to_lds<false>(make_rsrc(kl + r0, BLK * 256), 256, Ks, BLK, wave, NW, lane);
      tile_to_lds<true>(make_rsrc(vl + r0, BLK * 256), 256, Vs, BLK, wave, NW, lane);
      wait_vmem();
      __syncthreads();
      qk_tile<NT>(Ks, qreg, S, l32, hh);
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint32_t word = selm[(c * BLK) / 32 + t];
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const int kin = 8 * (x >> 2) + 4 * hh + (x & 3);
          const int j = c * BLK + 32 * t + kin;
          const bool ok = j < Nb && !((word >> kin) & 1u);
          const float lg = ok ? (j == Nb - 1 ? lgLast : lgB) : -INFINITY;
          S[t][x] = fmaf(S[t][x], cs, lg);
          mx = fmaxf(mx, S[t][x]);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m, mx);
      const float alpha = m == m_new ? 1.0f : __builtin_amdgcn_exp2f(m - m_new);
      m = m_new;
      lsum *= alpha;
      beta *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) O[dt] *= alpha;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int x = 8 * u + e;
            const int j = c * BLK + 32 * t + 8 * (x >> 2) + 4 * hh + (x & 3);
            const float p = __builtin_amdgcn_exp2f(S[t][x] - m);
            lsum += p;
            beta = fmaf(p, j == Nb - 1 ? invLast : invB, beta);
            P[t][u][e] = (__bf16)p;
          }
      pv_tile<NT>(Vs, P, O, hh, g16, l16);
      __syncthreads();
    }
  }

  // ---- phase 3: global first-order correction ------------------------------------------------
  if (do_tail && (dm.phases & 4)) {
    const __bf16* ht = reinterpret_cast<const __bf16*>(w.hbarT_lo) + (size_t)h * 128 * 128;
    tile_to_lds<false>(make_rsrc(ht, 128 * 256), 256, smem, 128, wave, NW, lane);
    wait_vmem();
    __syncthreads();
    f32x16 T[4];
    qk_tile<4>(smem, qreg, T, l32, hh);
    const float bt = (beta + __shfl_xor(beta, 32)) * dm.scale;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) O[dt] += bt * T[dt];
    __syncthreads();
  }

  // ---- epilogue ------------------------------------------------------------------------------
  const float inv_l = 1.0f / (lsum + __shfl_xor(lsum, 32));
  {
    // O^T[dt] element x: query 32*wave + l32, column d = 32 dt + 8 (x/4) + 4 hh + (x%4)
    const uint32_t q = 32 * wave + l32;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (__bf16)(O[dt][4 * g + r] * inv_l);
        const uint32_t byte = (32 * dt + 8 * g + 4 * hh) * 2;
        *reinterpret_cast<bf16x4*>(smem + q * 256 + swz_row(q, byte >> 4) * 16 + (byte & 15)) = v;
      }
  }
  __syncthreads();
  __bf16* orow = out + head + (size_t)i * B * 128;
  for (int e = tid; e < n_i * 16; e += BLK * 2) {
    const uint32_t q = e >> 4, c = e & 15;
    const u32x4 v = *reinterpret_cast<const u32x4*>(smem + q * 256 + swz_row(q, c) * 16);
    *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(orow) + q * 256 + c * 16) = v;
  }
}

}  // namespace

hipError_t launch_attend_bf16(const Dims& dm, const Work& w, const void* Q, const void* K, const void* V, void* out,
                              hipStream_t s) {
  const int items = dm.H * dm.Nb;
  auto q = static_cast<const __bf16*>(Q);
  auto k = static_cast<const __bf16*>(K);
  auto v = static_cast<const __bf16*>(V);
  auto o = static_cast<__bf16*>(out);
  if (dm.B == 128)
    hipLaunchKernelGGL(attend_bf16<128>, dim3(items), dim3(256), 0, s, dm, w, q, k, v, o);
  else
    hipLaunchKernelGGL(attend_bf16<64>, dim3(items), dim3(128), 0, s, dm, w, q, k, v, o);
  return hipGetLastError();
}

}  // namespace pisa
