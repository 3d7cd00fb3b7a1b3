// Internal interface between the C-ABI host layer (pisa_host.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace pisa {

// Most blocks whose K^T V products one statistics workgroup sums before writing a partial of
// H-bar (Dims::chunk is this, or less for layers too small to fill the chip with 16).
constexpr int kStatsChunk = 16;
// Most workgroups of the bf16 statistics passes (two resident per CU on 256 CUs: one round).
constexpr int kStatsWorkgroups = 512;

struct Dims {
  int H;
  int L;
  int d;
  int B;
  int Nb;      // ceil(L / B)
  int k;       // critical blocks per query block
  int n_last;  // rows of the last block
  int NC;      // ceil(Nb / chunk): partial H-bar sums per head
  int Nbp;     // Nb rounded up to a multiple of B (pooled-token tiles)
  float scale; // softmax scale applied to q
  int routing; // 0 covariance-aware, 1 plain
  int phases;  // bit mask: 1 exact, 2 zeroth order, 4 first order
  int dtype;   // 0 bf16, 1 fp32
  int first_block;  // 1: block-wise first-order term (per-block H_j) instead of H-bar
  int spectral;     // 1: M_j = spectral norm of H_j - H-bar (default Frobenius)
  int chunk;        // blocks per statistics workgroup (<= kStatsChunk; fp32 and per-block passes)
  int SW;           // workgroups of the bf16 statistics and Frobenius covariance passes
};

// The bf16 statistics and Frobenius covariance passes split the H * N_b (head, block) pairs, taken
// in head-major order g = h * N_b + j, into SW contiguous ranges whose lengths differ by at most one:
// range w is [stat_range_begin(w), stat_range_begin(w + 1)). A range may meet several heads; its
// partial sums for head h go to slot w + h. No two (range, head) pairs share a slot: a later range
// w' > w meets no head before the last head range w meets, so w' + h' > w + h. Head h's partials
// are the slots stat_owner(h N_b) + h .. stat_owner(h N_b + N_b - 1) + h.
__host__ __device__ inline int stat_range_begin(const Dims& dm, int w) {
  return (int)(((long long)w * dm.H * dm.Nb) / dm.SW);
}
// The range holding pair g (every range holds at least one pair: SW <= H * N_b).
__host__ __device__ inline int stat_owner(const Dims& dm, int g) {
  return (int)((((long long)g + 1) * dm.SW - 1) / ((long long)dm.H * dm.Nb));
}
// Partial slots of the bf16 statistics pass: at most SW + H - 1.
__host__ __device__ inline int stat_slots(const Dims& dm) { return dm.SW + dm.H - 1; }

// The block-wise first-order variant runs when it is requested and there is a first-order term.
__host__ __device__ inline bool block_first_order(const Dims& dm) {
  return dm.first_block && dm.k < dm.Nb && (dm.phases & 6) == 6;
}

// Device pointers into the attached workspace.
struct Work {
  float* qbar;      // [H][Nb][d]   pooled scaled queries (mean of scale*q over the block)
  float* kbar;      // [H][Nb][d]   key centroids
  float* vsum;      // [H][Nb][d]   value sums
  float* G;         // [slots][d][d] partial sums of H_j = K_j^T V_j - kbar_j (sum V_j)^T: fp32 path
                    // H * NC slots (slot h NC + c), bf16 path stat_slots (slot w + h)
  float* hbar;      // [H][d][d]    H-bar
  float* M;         // [H][Nb]      ||H_j - H-bar||_F
  float* kpart;     // [slots][d]   partial sums of the block centroids, slots as G (bf16 path only)
  float* kc;        // [H][d]       key centre: mean of the block centroids   (bf16 path only)
  void* kbar_lo;    // bf16 [H][Nbp][d] centroid minus the key centre, zero rows past Nb (bf16 path only)
  void* vbar_lo;    // bf16 [H][Nbp][d] value means, zero rows past Nb    (bf16 path only)
  void* hbarT_lo;   // bf16 [H][d][d]   transpose of H-bar                (bf16 path only)
  int32_t* idx;     // [H][Nb][k]   ascending critical block indices
  void* hjT_lo;     // bf16 [H][Nb][d][d] transposes of every H_j         (block first order only)
  float* opart;     // [H][L][d]    unnormalised exact + zeroth-order numerator (block first order)
  float* ml;        // [H][L][2]    softmax reference and denominator        (block first order)
};

struct Layout {
  size_t qbar, kbar, vsum, G, hbar, M, kpart, kc, kbar_lo, vbar_lo, hbarT_lo, idx, hjT_lo, opart, ml, total;
};

Layout workspace_layout(const Dims& dm);

// Size of the static workspace of pisa_forward_noalloc (a file-scope device array per GPU): the
// plans of every bundled workload fit (the largest, the Wan2.1-14B-like 720p layer, needs 91 MiB).
constexpr size_t kStaticWorkspaceBytes = size_t(96) << 20;

// Device address of that array on the stream's device (looked up once per device, then cached).
hipError_t static_workspace(hipStream_t stream, void** ptr);
Work workspace_pointers(const Dims& dm, void* base);

// Statistics (precompute), routing and the fused attention kernel launchers. Each returns the
// first HIP error of its launches.
hipError_t launch_stats_pass(const Dims& dm, const Work& w, const void* Q, const void* K,
                             const void* V, hipStream_t s);      // centroids, sums, K^T V partials
hipError_t launch_stats_finalize(const Dims& dm, const Work& w, hipStream_t s);  // H-bar, lo copies
hipError_t launch_stats_cov(const Dims& dm, const Work& w, const void* K, const void* V,
                            hipStream_t s);                       // M_j
hipError_t launch_route(const Dims& dm, const Work& w, hipStream_t s);
hipError_t launch_attend(const Dims& dm, const Work& w, const void* Q, const void* K,
                         const void* V, void* out, hipStream_t s);   // + block first order if set

// Per-dtype implementations.
hipError_t launch_stats_pass_bf16(const Dims&, const Work&, const void*, const void*, const void*, hipStream_t);
hipError_t launch_stats_cov_bf16(const Dims&, const Work&, const void*, const void*, hipStream_t);
hipError_t launch_stats_pass_f32(const Dims&, const Work&, const void*, const void*, const void*, hipStream_t);
hipError_t launch_stats_cov_f32(const Dims&, const Work&, const void*, const void*, hipStream_t);
hipError_t launch_attend_bf16(const Dims&, const Work&, const void*, const void*, const void*, void*, hipStream_t);
hipError_t launch_mfma_probe(int blocks, int iters, float* out, uint64_t* clk, hipStream_t s);
hipError_t launch_first_block_bf16(const Dims&, const Work&, const void*, void*, hipStream_t);
hipError_t launch_attend_f32(const Dims&, const Work&, const void*, const void*, const void*, void*, hipStream_t);

}  // namespace pisa
