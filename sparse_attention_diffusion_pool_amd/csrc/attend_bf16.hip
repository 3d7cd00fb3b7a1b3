// Fused piecewise attention, bf16 inputs, d = 128 (gist.science summary of the PISA paper,
// section 2 "Core algorithm" for what is computed and "Hardware implementation" for the phase
// structure: exact blocks, then aggregated block vectors at zeroth order, then the global
// first-order correction, all inside one online softmax).
//
// Work decomposition: one workgroup per (head, query block of BLK rows), BLK/32 waves; wave w owns
// query rows 32 w .. 32 w + 31 and all keys. Two workgroups share a CU (64 KB of LDS each), so the
// two waves on each SIMD belong to different workgroups: one's softmax overlaps the other's MFMAs.
//
// Everything is computed transposed so that per-query state lives in the lane owning the query
// (lane % 32; lanes l and l ^ 32 hold the two halves of the query's keys / output columns):
//   S^T = K Q^T      A = K rows from LDS (16 B reads), B = Q^T held in registers
//   O^T += V^T P^T   A = V^T via ds_read_b64_tr_b16 from the row-major V tile,
//                    B = P^T straight from the S^T accumulators (converted to bf16)
//   T^T = Hbar^T Q^T phase 3, same routine as S^T with H-bar^T as the tile
//
// Keys stream in steps of 64 through two LDS stages (K and V halves, 16 KB each): step s + 1 is
// copied global -> LDS (buffer loads, rows past the block end read as zero) while step s is
// computed. A key block of 128 rows takes two steps; the selected block list is staged in LDS.
// Softmax runs in the log2 domain: Q enters the MFMA as given, and one FMA per score turns the raw
// q.k into the exponent argument scale log2(e) q.k - m (m = the row's reference). The reference is
// moved only when a row's max grows by more than 2^8 (exact: numerator and denominator share the
// stale reference, and p <= 256 stays far inside fp32/bf16 range).
// Phase 2: pooled tokens (kbar_j, vbar_j) through the same steps; each token's bias (ln n_j, or
// -inf outside U_i, from the bit mask in LDS, or past N_b) enters through one MFMA that starts the
// score tile, so the softmax is the exact steps' own. beta (the sum of p / n_j) takes each pooled
// step's row sum over B, plus a correction for a ragged last block's token. Phase 3:
// O += (beta * scale) (q H-bar).
// Epilogue: out = O / l, rounded to bf16, staged through LDS for 16-byte row stores.
#include "dev_common.h"
#include "pisa_internal.h"

namespace pisa {
namespace {

constexpr int kMaskWords = (8192 + 128) / 32;  // N_b <= 8192, rounded up to a tile
constexpr float kLazy = 8.0f;                   // rescale threshold (log2 units)
constexpr float kSumHi = 4294967296.0f;         // 2^32: a step's row sum above this moves the reference
constexpr float kSumLo = 2.3283064365386963e-10f;  // 2^-32: ... or below this while nothing is summed

// Per-lane LDS read offsets, computed once (relative to a tile's first row r0, r0 % 16 == 0):
//   krd[s]: 16-byte row read of row r0 + l32, d-chunk 2 s + hh (row-read swizzle)
//   vrd[dt]: transpose read of rows r0 + 4 hh + l16/4, columns 32 dt + 16 g16 + 4 (l16 % 4)
//            (transpose-read swizzle); other key rows of the same lane differ by multiples of 4
struct LaneOffsets {
  uint32_t krd[8];
  uint32_t vrd[4];
};

// base: byte offset of the wave's first key row in a tile (a multiple of 16 rows: the swizzles
// only depend on the row modulo 16)
__device__ __forceinline__ LaneOffsets lane_offsets(uint32_t lane, uint32_t base = 0) {
  const uint32_t hh = lane >> 5, l32 = lane & 31, g16 = (lane >> 4) & 1, l16 = lane & 15;
  LaneOffsets o;
#pragma unroll
  for (int s = 0; s < 8; ++s) o.krd[s] = base + l32 * 256 + swz_row(l32, 2 * s + hh) * 16;
  const uint32_t dr = l16 >> 2;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const uint32_t byte = (32 * dt + 16 * g16 + 4 * (l16 & 3)) * 2;
    o.vrd[dt] = base + (4 * hh + dr) * 256 + swz_tr(dr, byte >> 4) * 16 + (byte & 15);
  }
  return o;
}

// S^T for NT key subtiles of 32 rows starting at row r0 (r0 % 16 == 0):
// S[t] = Tile[r0 + 32 t + l32][:] . Q^T
// The K-row reads run two d-chunks ahead of the MFMAs that use them, through an explicit ring of
// operand registers; the scheduling fences keep the compiler from sinking each read next to its
// MFMA (which would expose one LDS round trip per MFMA).
// With kAccumulate the products are added to S as the caller initialised it.
template <int NT, bool kAccumulate = false>
__device__ __forceinline__ void qk_tile(const char* tile, uint32_t r0, const bf16x8 qreg[8], f32x16 S[NT],
                                        const LaneOffsets& lo) {
  constexpr int kAhead = 2, kRing = kAhead + 1;
  bf16x8 a[kRing][NT];
  auto load = [&](int s) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
      a[s % kRing][t] = *reinterpret_cast<const bf16x8*>(tile + (r0 + 32 * t) * 256 + lo.krd[s]);
  };
  if constexpr (!kAccumulate) {
#pragma unroll
    for (int t = 0; t < NT; ++t) S[t] = f32x16{};
  }
#pragma unroll
  for (int s = 0; s < kAhead; ++s) load(s);
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    if (s + kAhead < 8) load(s + kAhead);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < NT; ++t) S[t] = mfma32(a[s % kRing][t], qreg[s], S[t]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// O^T[dt] += V^T P^T over NT key subtiles starting at key r0 (r0 % 4 == 0). MFMA groups are
// (dt, t) in that order; the transpose reads of a group are issued two groups ahead.
template <int NT>
__device__ __forceinline__ void pv_tile(const char* Vs, uint32_t r0, const bf16x8 P[NT][2], f32x16 O[4],
                                        const LaneOffsets& lo) {
  constexpr int kGroups = 4 * NT, kAhead = 2, kRing = kAhead + 1;
  i16x4 x[kRing][2], y[kRing][2];
  auto load = [&](int g) __attribute__((always_inline)) {
    const int dt = g / NT, t = g % NT;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const char* base = Vs + (r0 + 32 * t + 16 * u) * 256 + lo.vrd[dt];
      x[g % kRing][u] = lds_tr16(base);
      y[g % kRing][u] = lds_tr16(base + 8 * 256);
    }
  };
#pragma unroll
  for (int g = 0; g < kAhead; ++g) load(g);
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    if (g + kAhead < kGroups) load(g + kAhead);
    __builtin_amdgcn_sched_barrier(0);
    const int dt = g / NT, t = g % NT;
#pragma unroll
    for (int u = 0; u < 2; ++u) O[dt] = mfma32(join_tr(x[g % kRing][u], y[g % kRing][u]), P[t][u], O[dt]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Workgroup id -> work item. Workgroup ids go to the 8 XCDs round-robin and start roughly in id
// order; in each super-chunk of 8 * kRun consecutive ids, XCD x gets kRun consecutive items
// (neighbouring query blocks of one head: their selected key blocks overlap, so they share the
// XCD's L2), and all XCDs work on the same head at a time (its K and V stay in the last-level
// cache).
constexpr int kRun = 64;
__device__ __forceinline__ int item_of(int bid, int n) {
  constexpr int chunk = 8 * kRun;
  const int g = bid / chunk, r = bid % chunk;
  if (g >= n / chunk) return bid;
  return g * chunk + (r % 8) * kRun + r / 8;
}

template <int V>
struct Stage {
  static constexpr int value = V;
};

constexpr int kKT = 64;           // keys per step
constexpr int kIdxLds = 4096;     // selected-block list entries staged in LDS

template <int BLK>
__global__ __launch_bounds__(256, 2) void attend_bf16(Dims dm, Work w, const __bf16* __restrict__ Q,
                                                      const __bf16* __restrict__ K,
                                                      const __bf16* __restrict__ V,
                                                      __bf16* __restrict__ out) {
  constexpr int NW = 4;            // waves
  constexpr int KS = 128 / BLK;    // waves per query group: each takes 1/KS of every step's keys
  constexpr int QG = NW / KS;      // query groups of 32 rows
  constexpr int NTH = 64 * NW;
  constexpr int SPB = BLK / kKT;   // steps per key block (and per pooled tile)
  constexpr int NT = kKT / 32 / KS;  // 32-key subtiles per wave and step
  constexpr int TB = kKT * 256;    // bytes of one K (or V) half
  // Two stages (K and V halves) as four distinct LDS objects: the compiler then sees that reading
  // one stage does not depend on the direct-to-LDS copies into the other.
  __shared__ __attribute__((aligned(1024))) char sK0[TB];
  __shared__ __attribute__((aligned(1024))) char sK1[TB];
  __shared__ __attribute__((aligned(1024))) char sV0[TB];
  __shared__ __attribute__((aligned(1024))) char sV1[TB];
  __shared__ uint32_t selm[kMaskWords];
  __shared__ uint16_t sidx[kIdxLds];

  const int item = item_of(blockIdx.x, gridDim.x);
  // (the divisions run on the vector unit: readfirstlane keeps the results, and every address
  // derived from them, in scalar registers)
  const int h = __builtin_amdgcn_readfirstlane(item / dm.Nb), i = __builtin_amdgcn_readfirstlane(item % dm.Nb);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: LDS bases stay scalar
  // query group qg (rows 32 qg ..), key part kh: with B = 64 a query group is two waves, each
  // running its own online softmax over one half of every step's keys, merged at the end
  const int qg = KS == 1 ? wave : wave % QG, kh = KS == 1 ? 0 : wave / QG;
  const uint32_t hh = lane >> 5, l32 = lane & 31;
  const int Nb = dm.Nb, B = dm.B, kk = dm.k;
  const int n_i = (i == Nb - 1) ? dm.n_last : B;
  const size_t head = (size_t)h * dm.L * 128;
  const int32_t* sel = w.idx + ((size_t)h * Nb + i) * kk;
  const bool do_tail = kk < Nb && (dm.phases & 2);
  const bool do_first = do_tail && (dm.phases & 4) && !dm.first_block;
  const bool block_fo = block_first_order(dm);  // per-block first order: finished by first_block_bf16
  // pooled steps: the kKT-token tiles that hold a pooled token j < N_b (tokens past N_b are zero)
  const int nc = do_tail ? (Nb + kKT - 1) / kKT : 0;
  const __bf16* kl = reinterpret_cast<const __bf16*>(w.kbar_lo) + (size_t)h * dm.Nbp * 128;
  const __bf16* vl = reinterpret_cast<const __bf16*>(w.vbar_lo) + (size_t)h * dm.Nbp * 128;
  const __bf16* ht = reinterpret_cast<const __bf16*>(w.hbarT_lo) + (size_t)h * 128 * 128;

  // selection: bit mask (pooled tiles) and the list (exact steps) in LDS
  const int nmask = (dm.Nbp + 31) / 32;
  for (int t = tid; t < nmask; t += NTH) selm[t] = 0u;
  __syncthreads();
  for (int t = tid; t < kk; t += NTH) {
    const int j = sel[t];
    if (t < kIdxLds) sidx[t] = (uint16_t)j;
    atomicOr(&selm[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  auto block_raw = [&](int t) -> int {  // t-th selected block (uniform, held per lane)
    return kk <= kIdxLds ? (int)sidx[t] : sel[t];
  };

  // Steps: exact (two per 128-row block; the ragged last block, which is last if selected, drops
  // its second half when n_last <= 64), then pooled tiles, then the H-bar^T tile (128 rows over
  // both arrays of a stage).
  const int last_blk = __builtin_amdgcn_readfirstlane(block_raw(kk - 1));
  const int rows_last = last_blk == Nb - 1 ? dm.n_last : B;
  const int E = (kk - 1) * SPB + (rows_last + kKT - 1) / kKT;  // exact steps
  const bool ragged = (rows_last % kKT) != 0;                   // last exact step is partial
  const int S_main = E + nc;
  const int S_all = S_main + (do_first ? 1 : 0);

  // Byte offsets inside Q, K and V fit in 32 bits (the plan keeps H L d below 2^31 elements).
  const char* Kh = reinterpret_cast<const char*>(K + head);
  const char* Vh = reinterpret_cast<const char*>(V + head);
  const uint32_t cl_row = chunk_lane<false>(lane), cl_tr = chunk_lane<true>(lane);
  auto issue = [&](int s, auto stc) {
    constexpr int ST = decltype(stc)::value;
    const uint32_t Ks = lds_addr(ST ? sK1 : sK0), Vs = lds_addr(ST ? sV1 : sV0);
    if (s < E) {
      const int j = __builtin_amdgcn_readfirstlane(block_raw(s / SPB));
      const int r0 = kKT * (s % SPB);
      const int n_j = (j == Nb - 1) ? dm.n_last : B;
      const uint32_t off = ((uint32_t)j * (uint32_t)B + (uint32_t)r0) * 256u;
      const uint32_t bytes = (uint32_t)(n_j - r0) * 256;  // rows past the block end read as zero
      copy_tile_chunks<kKT, NW, false>(Kh + off, bytes, Ks, cl_row, wave);
      copy_tile_chunks<kKT, NW, true>(Vh + off, bytes, Vs, cl_tr, wave);
    } else if (s < S_main) {
      const size_t g0 = (size_t)(s - E) * kKT * 128;
      copy_tile_chunks<kKT, NW, false>(kl + g0, kKT * 256, Ks, cl_row, wave);
      copy_tile_chunks<kKT, NW, true>(vl + g0, kKT * 256, Vs, cl_tr, wave);
    } else {
      copy_tile_chunks<kKT, NW, false>(ht, kKT * 256, Ks, cl_row, wave);
      copy_tile_chunks<kKT, NW, false>(ht + kKT * 128, kKT * 256, Vs, cl_row, wave);
    }
  };
  issue(0, Stage<0>{});

  // Q^T operand: query row 32 qg + l32 of the block, d = 16 s + 8 hh .. +7
  bf16x8 qreg[8];
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + head + (size_t)i * B * 128, n_i * 256);
    const uint32_t row = 32 * qg + l32;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      qreg[s] = __builtin_bit_cast(bf16x8, buf_load16(rq, row * 256 + (16 * s + 8 * hh) * 2));
  }
  // Q stays as given (exact bf16): the MFMA gives raw q.k in fp32, and the softmax scale (times
  // log2 e) is applied in fp32 by one FMA per score, x = cs q.k - m. Rounding cs q to bf16 instead
  // would add an error of up to 2^-9 |cs q.k| to every exponent, which sharp score distributions
  // (spreads of 6 and more) turn into output errors above the bf16 tolerance.
  const float cs = dm.scale * kLog2e;
  // The pooled centroids are stored relative to the head's key centre c: their scores get
  // cs q.c back through the FMA's addend (q.c in fp32, over the lane's half of d, then the pair).
  float csqc = 0.f;
  if (nc > 0) {
    const float* kcen = w.kc + (size_t)h * 128;
    float a = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const f32x4 c0 = *reinterpret_cast<const f32x4*>(kcen + 16 * s + 8 * hh);
      const f32x4 c1 = *reinterpret_cast<const f32x4*>(kcen + 16 * s + 8 * hh + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a = fmaf((float)qreg[s][e], c0[e], a);
        a = fmaf((float)qreg[s][e + 4], c1[e], a);
      }
    }
    csqc = cs * (a + __shfl_xor(a, 32));
  }
  // Operands of the bias MFMA that starts every pooled score tile, D[key][q] = sum over k < 3 of
  // A[key][k] B[k][q] with B rows 1 and 2 = 1: A columns 1 and 2 hold the token's bias in raw score
  // units, log2(n_j) / cs split into a bf16 head and tail, or -inf for a selected block or j >= N_b.
  bf16x8 shift_b = {};
  shift_b[1] = (__bf16)(hh == 0 ? 1.0f : 0.0f);
  shift_b[2] = shift_b[1];
  const float bB = __log2f((float)B) / cs, bLast = __log2f((float)dm.n_last) / cs;
  const __bf16 bB_hi = (__bf16)bB, bB_lo = (__bf16)(bB - (float)bB_hi);
  const __bf16 bLast_hi = (__bf16)bLast, bLast_lo = (__bf16)(bLast - (float)bLast_hi);
  const float invB = 1.0f / (float)B;
  // beta takes a pooled step's row sum over B. For a ragged last block (n_last < B) the step that
  // holds its token (s_last) adds p (1 / n_last - 1 / B), with p read from the token's accumulator:
  // key row i = (N_b - 1) % 32 of subtile u_last, in lanes with hh = (i / 4) % 2, element
  // (i % 4) + 4 (i / 8).
  const int s_last = dm.n_last != B ? E + (Nb - 1) / kKT : -1;
  const int r_last = (Nb - 1) % kKT, i_last = r_last % 32;
  const int u_last = r_last / 32, hh_last = (i_last / 4) % 2, x_last = (i_last % 4) + 4 * (i_last / 8);
  const float corr_last = 1.0f / (float)dm.n_last - invB;
  // m: the row's softmax reference (log2 units), 0 until a step moves it; neg_m = -m
  float m = 0.f, neg_m = 0.f, lsum = 0.f, beta = 0.f;
  f32x16 O[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) O[dt] = f32x16{};
  const LaneOffsets lofs = lane_offsets(lane, (uint32_t)(32 * NT * kh) * 256u);
  // The two waves sharing a SIMD come from different workgroups. A fixed priority order between
  // them (by the parity of the hardware wave slot, HW_ID bits 0..3) lets one run at its own pace
  // while the other fills its gaps, instead of both competing for every issue slot.
  if (__builtin_amdgcn_s_getreg((4 << 0) | (0 << 6) | (3 << 11)) & 1) __builtin_amdgcn_s_setprio(2);

  // One step s (ST = s & 1). KIND 0 = exact, 1 = exact partial (masked past valid rows), 2 = pooled.
  // The reference m is not moved step by step: the probabilities are formed against it as it
  // stands, and only a step whose row sum leaves [2^-32 (while nothing has been summed), 2^32]
  // (or is not finite) takes the rare path that recomputes the step's scores and moves m to the
  // row's maximum. Every probability then stays below 2^32 (far inside fp32 and bf16 range), and
  // numerator and denominator always share the reference.
  auto step = [&](int s, auto stc, auto kc) {
    constexpr int ST = decltype(stc)::value;
    constexpr int KIND = decltype(kc)::value;
    wait_vmem();
    __syncthreads();  // step s landed; step s - 1 no longer read by anyone
    if (s + 1 < S_all) issue(s + 1, Stage<ST ^ 1>{});
    f32x16 Sc[NT];
    bf16x8 P[NT][2];
    float s_tok = -INFINITY;
    // Exact tiles start from zero; pooled tiles from the bias MFMA. After the products, one FMA per
    // score gives the exponent argument x = cs (q.k + bias) - m (pooled: q.(kbar_j - c) + cs q.c).
    auto scores = [&]() __attribute__((always_inline)) {
      if constexpr (KIND == 2) {
        // A row = key l32 of subtile t: pooled token j = (s - E) kKT + 32 (NT kh + t) + l32
        const int key_base = (s - E) * kKT + 32 * NT * kh;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int j = key_base + 32 * t + (int)l32;
          const bool sel_j = (selm[(key_base + 32 * t) / 32] >> l32) & 1u;
          const bool ok = j < Nb && !sel_j && hh == 0;
          const bool last = j == Nb - 1;
          bf16x8 a = {};
          a[1] = ok ? (last ? bLast_hi : bB_hi) : (__bf16)(hh == 0 ? -INFINITY : 0.0f);
          a[2] = ok ? (last ? bLast_lo : bB_lo) : (__bf16)0.0f;
          Sc[t] = mfma32(a, shift_b, f32x16{});
        }
        qk_tile<NT, true>(ST ? sK1 : sK0, 0, qreg, Sc, lofs);
      } else {
        qk_tile<NT, false>(ST ? sK1 : sK0, 0, qreg, Sc, lofs);
      }
      const float add = KIND == 2 ? neg_m + csqc : neg_m;
#pragma unroll
      for (int u = 0; u < NT; ++u)
#pragma unroll
        for (int x = 0; x < 16; ++x) Sc[u][x] = fmaf(Sc[u][x], cs, add);
      if constexpr (KIND == 1) {
        // key 32 u + 8 (x / 4) + 4 hh + x % 4 of this lane is masked when it reaches the step's
        // valid rows; comparing the constant part with (valid - 4 hh) keeps the key indices out of
        // registers
        const int vrel = rows_last - kKT * ((E - 1) % SPB) - 32 * NT * kh - 4 * (int)hh;
#pragma unroll
        for (int u = 0; u < NT; ++u)
#pragma unroll
          for (int x = 0; x < 16; ++x)
            if (32 * u + 8 * (x >> 2) + (x & 3) >= vrel) Sc[u][x] = -INFINITY;
      }
    };
    // probabilities (rounded to bf16: the values the numerator's MFMA uses) and their sum over the
    // lane's keys, in four independent dot2 chains; the ragged last block's pooled token score is
    // taken first (wave-uniform branch)
    auto probs = [&]() __attribute__((always_inline)) {
      if constexpr (KIND == 2) {
        if (s == s_last && u_last / NT == kh) {
          s_tok = Sc[0][x_last];
#pragma unroll
          for (int u = 1; u < NT; ++u)
            if (u == u_last % NT) s_tok = Sc[u][x_last];
        }
      }
#pragma unroll
      for (int u = 0; u < NT; ++u)
#pragma unroll
        for (int v = 0; v < 2; ++v)
#pragma unroll
          for (int e = 0; e < 8; ++e) P[u][v][e] = (__bf16)__builtin_amdgcn_exp2f(Sc[u][8 * v + e]);
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
      float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < NT; ++u)
#pragma unroll
        for (int v = 0; v < 2; ++v)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            part[e] = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{P[u][v][2 * e], P[u][v][2 * e + 1]}, ones, part[e],
                                                      false);
      return (part[0] + part[1]) + (part[2] + part[3]);
    };
    scores();
    float ps = probs();
    const bool bad = !(ps <= kSumHi) || (lsum == 0.0f && ps < kSumLo);
    if (__builtin_expect(__ballot(bad) != 0, 0)) {
      // rare: the step's scores again (the tile is still in LDS), and the reference of every row
      // whose maximum is above 2^8 or that has nothing summed yet moves to that maximum
      scores();
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < NT; ++u)
#pragma unroll
        for (int x = 0; x < 16; ++x) mx = fmaxf(mx, Sc[u][x]);
      mx = xor32_max(mx);
      const float lrow = lsum + __shfl_xor(lsum, 32);
      const bool up = mx > -INFINITY && (mx > kLazy || lrow == 0.0f);
      const float shift = up ? mx : 0.0f;
      const float alpha = __builtin_amdgcn_exp2f(-shift);
      m += shift;
      neg_m = -m;
      lsum *= alpha;
      beta *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) O[dt] *= alpha;
#pragma unroll
      for (int u = 0; u < NT; ++u) Sc[u] -= shift;
      ps = probs();
    }
    lsum += ps;
    if constexpr (KIND == 2) {
      // a pooled step's sum, divided by the block size, also feeds beta
      beta = fmaf(ps, invB, beta);
      if (s == s_last && (int)hh == hh_last) beta = fmaf(__builtin_amdgcn_exp2f(s_tok), corr_last, beta);
    }
    pv_tile<NT>(ST ? sV1 : sV0, 0, P, O, lofs);
  };

  const int E_full = E - (ragged ? 1 : 0);
  int s0 = 0;
  for (; s0 + 1 < E_full; s0 += 2) {
    step(s0, Stage<0>{}, Stage<0>{});
    step(s0 + 1, Stage<1>{}, Stage<0>{});
  }
  if (s0 < E_full) step(s0, Stage<0>{}, Stage<0>{});
  if (ragged) {
    if (E_full & 1)
      step(E_full, Stage<1>{}, Stage<1>{});
    else
      step(E_full, Stage<0>{}, Stage<1>{});
  }
  for (int s = E; s < S_main; ++s) {
    if (s & 1)
      step(s, Stage<1>{}, Stage<2>{});
    else
      step(s, Stage<0>{}, Stage<2>{});
  }

  lsum += __shfl_xor(lsum, 32);
  beta += __shfl_xor(beta, 32);
  wait_vmem();
  __syncthreads();  // every wave done with the last step; the H-bar^T tile (if any) has landed
  const int hstage = S_main & 1;
  const int xs = do_first ? (hstage ^ 1) : 0;  // the stage free for exchanges and output staging
  if constexpr (KS == 2) {
    // merge the two key halves of each query group: the kh = 1 wave hands its reference,
    // denominator, beta and numerator to the kh = 0 wave through LDS (numerators in the free
    // stage, one array per group; the scalars in the selection list's space, no longer read)
    float* xo = reinterpret_cast<float*>(qg == 0 ? (xs ? sK1 : sK0) : (xs ? sV1 : sV0));
    float* xm = reinterpret_cast<float*>(sidx) + qg * 3 * 64;
    if (kh == 1) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int x = 0; x < 16; ++x) xo[(dt * 16 + x) * 64 + lane] = O[dt][x];
      xm[lane] = m;
      xm[64 + lane] = lsum;
      xm[128 + lane] = beta;
    }
    __syncthreads();
    if (kh == 0) {
      const float mp = xm[lane], lp = xm[64 + lane], bp = xm[128 + lane];
      const float mm = fmaxf(m, mp);
      const float a0 = __builtin_amdgcn_exp2f(m - mm), a1 = __builtin_amdgcn_exp2f(mp - mm);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int x = 0; x < 16; ++x) O[dt][x] = fmaf(a1, xo[(dt * 16 + x) * 64 + lane], a0 * O[dt][x]);
      m = mm;
      lsum = fmaf(a1, lp, a0 * lsum);
      beta = fmaf(a1, bp, a0 * beta);
    }
    __syncthreads();  // the exchange is read before the stage is reused for the output rows
  }
  const bool owner = kh == 0;  // the waves that finish and store the rows
  // ---- phase 3: global first-order correction --------------------------------------------
  if (do_first && owner) {
    f32x16 T2[2];
    const float bt = beta * dm.scale;
    qk_tile<2>(hstage ? sK1 : sK0, 0, qreg, T2, lofs);  // H-bar^T rows 0..63
    O[0] += bt * T2[0];
    O[1] += bt * T2[1];
    qk_tile<2>(hstage ? sV1 : sV0, 0, qreg, T2, lofs);  // H-bar^T rows 64..127
    O[2] += bt * T2[0];
    O[3] += bt * T2[1];
  }
  if (block_fo) {
    // hand the unnormalised numerator and (reference, denominator) to the block first-order kernel
    const uint32_t q = 32 * qg + l32;
    if (owner && (int)q < n_i) {
      const size_t row = (size_t)h * dm.L + (size_t)i * B + q;
      float* orow = w.opart + row * 128;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 v = {O[dt][4 * g], O[dt][4 * g + 1], O[dt][4 * g + 2], O[dt][4 * g + 3]};
          *reinterpret_cast<f32x4*>(orow + 32 * dt + 8 * g + 4 * hh) = v;
        }
      if (hh == 0) {
        w.ml[2 * row] = m == -INFINITY ? 0.0f : m;
        w.ml[2 * row + 1] = lsum;
      }
    }
    return;
  }
  // ---- epilogue: bf16 output rows via LDS (queries 0..63 in one array, 64..127 in the other) --
  char* stg_lo = xs ? sK1 : sK0;
  char* stg_hi = xs ? sV1 : sV0;
  const float inv_l = 1.0f / lsum;
  if (owner) {
    const uint32_t q = 32 * qg + l32;
    char* stg = q < 64 ? stg_lo : stg_hi;
    const uint32_t qr = q & 63;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (__bf16)(O[dt][4 * g + r] * inv_l);
        const uint32_t byte = (32 * dt + 8 * g + 4 * hh) * 2;
        *reinterpret_cast<bf16x4*>(stg + qr * 256 + swz_row(qr, byte >> 4) * 16 + (byte & 15)) = v;
      }
  }
  __syncthreads();
  __bf16* orow = out + head + (size_t)i * B * 128;
  for (int e = tid; e < n_i * 16; e += NTH) {
    const uint32_t q = e >> 4, c = e & 15;
    const char* stg = q < 64 ? stg_lo : stg_hi;
    const uint32_t qr = q & 63;
    const u32x4 v = *reinterpret_cast<const u32x4*>(stg + qr * 256 + swz_row(qr, c) * 16);
    *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(orow) + q * 256 + c * 16) = v;
  }
}

// Block-wise first-order variant (an ablation of the global H-bar term): for every unselected
// block j of the query block, O^T += (alpha_{t,j} scale) (H_j^T Q^T), with alpha_{t,j} relative to
// the softmax reference the attention kernel used, then out = O / l. One workgroup per (head,
// query block), BLK/32 waves of 32 queries; H_j^T (bf16, 32 KB) and the centroid row stream
// through two LDS stages; q . kbar_j is a per-lane dot product over the lane's half of d.
template <int BLK>
__global__ __launch_bounds__(BLK * 2, 1) void first_block_bf16(Dims dm, Work w, const __bf16* __restrict__ Q,
                                                               __bf16* __restrict__ out) {
  constexpr int NW = BLK / 32;
  constexpr int NTH = 64 * NW;
  constexpr int TB = 64 * 256;  // half of H_j^T: 64 rows of 128 bf16
  __shared__ __attribute__((aligned(1024))) char sA0[TB];
  __shared__ __attribute__((aligned(1024))) char sB0[TB];
  __shared__ __attribute__((aligned(1024))) char sA1[TB];
  __shared__ __attribute__((aligned(1024))) char sB1[TB];
  __shared__ __attribute__((aligned(1024))) char sk0[1024];  // centroid rows j .. j + 3 (row j used)
  __shared__ __attribute__((aligned(1024))) char sk1[1024];
  __shared__ uint32_t selm[kMaskWords];
  __shared__ uint16_t uidx[8192];

  const int item = blockIdx.x;
  const int h = item / dm.Nb, i = item % dm.Nb;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t hh = lane >> 5, l32 = lane & 31;
  const int Nb = dm.Nb, B = dm.B, kk = dm.k;
  const int n_i = (i == Nb - 1) ? dm.n_last : B;
  const size_t head = (size_t)h * dm.L * 128;
  const int32_t* sel = w.idx + ((size_t)h * Nb + i) * kk;
  const __bf16* hjt = reinterpret_cast<const __bf16*>(w.hjT_lo) + (size_t)h * Nb * 128 * 128;
  const __bf16* kl = reinterpret_cast<const __bf16*>(w.kbar_lo) + (size_t)h * dm.Nbp * 128;

  // U_i in ascending order: mark S_i, then wave 0 compacts the unmarked blocks with ballots
  const int nmask = (Nb + 31) / 32;
  for (int t = tid; t < nmask; t += NTH) selm[t] = 0u;
  __syncthreads();
  for (int t = tid; t < kk; t += NTH) {
    const int j = sel[t];
    atomicOr(&selm[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  if (wave == 0) {
    int base = 0;
    for (int j0 = 0; j0 < Nb; j0 += 64) {
      const int j = j0 + lane;
      const bool in_u = j < Nb && !((selm[j >> 5] >> (j & 31)) & 1u);
      const uint64_t bal = __ballot(in_u);
      const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
      if (in_u) uidx[base + before] = (uint16_t)j;
      base += __popcll(bal);
    }
  }
  __syncthreads();
  const int nU = Nb - kk;

  const uint32_t vb_row = copy_vbase<false>(wave, lane), vb_row2 = copy_vbase<false>(wave, lane, 8);
  auto issue = [&](int u, auto stc) {
    constexpr int ST = decltype(stc)::value;
    const int j = __builtin_amdgcn_readfirstlane((int)uidx[u]);
    const __bf16* src = hjt + (size_t)j * 128 * 128;
    copy_tile<64, NW>(make_rsrc(src, TB), ST ? sA1 : sA0, vb_row, wave, vb_row2);
    copy_tile<64, NW>(make_rsrc(src + 64 * 128, TB), ST ? sB1 : sB0, vb_row, wave, vb_row2);
    if (wave == 0) buf_load_lds16(make_rsrc(kl + (size_t)j * 128, (uint32_t)(dm.Nbp - j) * 256), ST ? sk1 : sk0, lane * 16);
  };
  issue(0, Stage<0>{});

  bf16x8 qreg[8];
  const uint32_t q = 32 * wave + l32;
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + head + (size_t)i * B * 128, n_i * 256);
#pragma unroll
    for (int s = 0; s < 8; ++s)
      qreg[s] = __builtin_bit_cast(bf16x8, buf_load16(rq, q * 256 + (16 * s + 8 * hh) * 2));
  }
  // numerator (exact + zeroth order), reference and denominator from the attention kernel
  const size_t row0 = (size_t)h * dm.L + (size_t)i * B;
  f32x16 O[4];
  {
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(w.opart + row0 * 128, n_i * 512);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x4 v = buf_load16(ro, q * 512 + (32 * dt + 8 * g + 4 * hh) * 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) O[dt][4 * g + r] = __uint_as_float(v[r]);
      }
  }
  float mref = 0.f, lsum = 1.f;
  if ((int)q < n_i) {
    mref = w.ml[2 * (row0 + q)];
    lsum = w.ml[2 * (row0 + q) + 1];
  }
  const float cs = dm.scale * kLog2e;
  const LaneOffsets lofs = lane_offsets(lane);
  // q.c, c = the key centre the pooled centroids are stored relative to
  float qc = 0.f;
  {
    const float* kcen = w.kc + (size_t)h * 128;
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) qc = fmaf((float)qreg[s][e], kcen[16 * s + 8 * hh + e], qc);
    qc += __shfl_xor(qc, 32);
  }

  auto step = [&](int u, auto stc) {
    constexpr int ST = decltype(stc)::value;
    wait_vmem();
    __syncthreads();  // stage ST landed; the other stage is free
    if (u + 1 < nU) issue(u + 1, Stage<ST ^ 1>{});
    // a = q . kbar_j over this lane's half of d, then across the lane pair
    const char* kr = ST ? sk1 : sk0;
    float a = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 kv = *reinterpret_cast<const bf16x8*>(kr + (16 * s + 8 * hh) * 2);
#pragma unroll
      for (int e = 0; e < 8; ++e) a = fmaf((float)qreg[s][e], (float)kv[e], a);
    }
    a += __shfl_xor(a, 32) + qc;
    const float wgt = __builtin_amdgcn_exp2f(fmaf(a, cs, -mref)) * dm.scale;
    f32x16 T[2];
    qk_tile<2>(ST ? sA1 : sA0, 0, qreg, T, lofs);  // (q H_j)[0..63]
    O[0] += wgt * T[0];
    O[1] += wgt * T[1];
    qk_tile<2>(ST ? sB1 : sB0, 0, qreg, T, lofs);  // (q H_j)[64..127]
    O[2] += wgt * T[0];
    O[3] += wgt * T[1];
  };
  int u = 0;
  for (; u + 1 < nU; u += 2) {
    step(u, Stage<0>{});
    step(u + 1, Stage<1>{});
  }
  if (u < nU) step(u, Stage<0>{});
  __syncthreads();  // every wave done with the stages: reuse them for the output rows

  char* stg_lo = sA0;
  char* stg_hi = sB0;
  const float inv_l = 1.0f / lsum;
  {
    char* stg = q < 64 ? stg_lo : stg_hi;
    const uint32_t qr = q & 63;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (__bf16)(O[dt][4 * g + r] * inv_l);
        const uint32_t byte = (32 * dt + 8 * g + 4 * hh) * 2;
        *reinterpret_cast<bf16x4*>(stg + qr * 256 + swz_row(qr, byte >> 4) * 16 + (byte & 15)) = v;
      }
  }
  __syncthreads();
  __bf16* orow = out + head + (size_t)i * B * 128;
  for (int e = tid; e < n_i * 16; e += NTH) {
    const uint32_t qq = e >> 4, c = e & 15;
    const char* stg = qq < 64 ? stg_lo : stg_hi;
    const uint32_t qr = qq & 63;
    const u32x4 v = *reinterpret_cast<const u32x4*>(stg + qr * 256 + swz_row(qr, c) * 16);
    *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(orow) + qq * 256 + c * 16) = v;
  }
}

}  // namespace

hipError_t launch_first_block_bf16(const Dims& dm, const Work& w, const void* Q, void* out, hipStream_t s) {
  const int items = dm.H * dm.Nb;
  auto q = static_cast<const __bf16*>(Q);
  auto o = static_cast<__bf16*>(out);
  if (dm.B == 128)
    hipLaunchKernelGGL(first_block_bf16<128>, dim3(items), dim3(256), 0, s, dm, w, q, o);
  else
    hipLaunchKernelGGL(first_block_bf16<64>, dim3(items), dim3(128), 0, s, dm, w, q, o);
  return hipGetLastError();
}

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
    hipLaunchKernelGGL(attend_bf16<64>, dim3(items), dim3(256), 0, s, dm, w, q, k, v, o);
  return hipGetLastError();
}

}  // namespace pisa
