/*
 * libpisa - PISA piecewise sparse attention, forward pass, for AMD Instinct MI355X (gfx950).
 *
 * The operation (per batch-head; the pages describing "PISA: Piecewise Sparse Attention Is Wiser
 * for Efficient Diffusion Transformers"):
 *   - Q, K, V are cut into blocks of B rows (AI Radio episode, paper summary; gist.science
 *     technical summary, section 2 "Core algorithm"). Query block i keeps a critical set S_i of k
 *     key/value blocks, computed exactly; the other blocks U_i are approximated.
 *   - Precompute (gist.science section 2 "Hardware implementation"): per block the key centroid
 *     kbar_j, the value sum, the block first-order matrix H_j = sum_n (k_n - kbar_j)^T v_n, their
 *     mean H-bar over all blocks, and M_j = ||H_j - H-bar|| for routing (section 2
 *     "Covariance-aware routing"; Frobenius norm by default, spectral as an option).
 *   - Routing: S_i = the k largest Score_{i,j} = qbar_i . kbar_j + ln(n_j + ||qbar_i|| M_j)
 *     (qbar_i = mean scaled query of block i; ties to the lower j). The pages name the score's
 *     ingredients but print no formula: this is the library's reading (PISA_ROUTING_PLAIN drops
 *     the covariance term).
 *   - Output (gist.science section 2 "Core algorithm", numerator formula): o_t = N_t / D_t with
 *       N_t = sum_{j in S_i} sum_n e^{q~_t.k_n} v_n + sum_{j in U_i} alpha_{t,j} sum_n v_{j,n}
 *             + beta_t (q~_t H-bar),       alpha_{t,j} = e^{q~_t.kbar_j},  beta_t = sum_U alpha
 *       D_t = sum_{j in S_i} sum_n e^{q~_t.k_n} + sum_{j in U_i} n_j alpha_{t,j}
 *     q~ = scale * q (default scale 1/sqrt(d)). D_t has no first-order part because kbar_j is
 *     the block mean.
 *
 * Layout: Q, K, V and out are contiguous [H, L, d] (batch folded into H: every statistic is per
 * batch-head), row-major, all of one dtype (bf16 or fp32), 16-byte aligned device pointers. out
 * must not overlap Q, K or V. A ragged last block (L % B != 0) is handled.
 *
 * Ownership: the caller owns Q, K, V, out and the workspace (device memory attached with
 * pisa_plan_attach_workspace); the plan owns host state only. pisa_plan/_set/_info/_destroy make
 * no HIP call. pisa_forward* enqueue kernels on `stream` and return without synchronising; a plan
 * (its workspace) must not be used by two calls that can run concurrently.
 *
 * Errors: every call returns a pisa_status and never aborts. Argument errors are reported before
 * any launch: NULL, misaligned or overlapping pointers first (no HIP call), then, once a device is
 * present, any of Q, K, V, out or the workspace that is not device memory (a host address) or
 * whose extent runs past the end of its allocation. A failed launch or missing device returns
 * PISA_ERR_DEVICE. pisa_last_error() gives the calling thread's last error text.
 *
 * Supported: dtype bf16 with d = 128, B in {64, 128}; dtype fp32 with d in {64, 128},
 * B in {64, 128}; L >= 1, H >= 1, 0 < keep <= 1, H * L * d < 2^31 elements per tensor;
 * N_b <= 8192.
 */
#ifndef PISA_H_
#define PISA_H_

#include <stddef.h>
#include <stdint.h>
/* hipStream_t comes from the HIP runtime header, which needs its platform named; a C or C++
 * consumer compiled without hipcc (gcc, clang) gets the AMD platform here. */
#ifndef __HIP_PLATFORM_AMD__
#define __HIP_PLATFORM_AMD__ 1
#endif
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pisa_plan_s pisa_plan_t;

typedef enum pisa_status {
  PISA_OK = 0,
  PISA_ERR_INVALID_ARGUMENT = 1, /* bad size, option value or pointer */
  PISA_ERR_UNSUPPORTED = 2,      /* valid but not implemented (d, B, dtype combination) */
  PISA_ERR_INVALID_HANDLE = 3,   /* NULL or destroyed plan */
  PISA_ERR_WORKSPACE = 4,        /* no workspace attached, too small or misaligned */
  PISA_ERR_DEVICE = 5            /* no HIP device, or a HIP call / kernel launch failed */
} pisa_status;

typedef enum pisa_option {
  PISA_OPT_DTYPE = 0,   /* PISA_DTYPE_BF16 (default for d = 128) or PISA_DTYPE_F32 (default otherwise) */
  PISA_OPT_SCALE = 1,   /* softmax scale tau > 0 applied to q (default 1/sqrt(d)) */
  PISA_OPT_ROUTING = 2, /* PISA_ROUTING_COV (default) or PISA_ROUTING_PLAIN */
  PISA_OPT_PHASES = 3,  /* bit mask of PISA_PHASE_* (default all three); EXACT must be set */
  PISA_OPT_FIRST_ORDER = 4, /* PISA_FIRST_ORDER_GLOBAL (default) or PISA_FIRST_ORDER_BLOCK */
  PISA_OPT_NORM = 5         /* matrix norm in M_j: PISA_NORM_FROBENIUS (default) or PISA_NORM_SPECTRAL */
} pisa_option;

enum { PISA_DTYPE_BF16 = 0, PISA_DTYPE_F32 = 1 };
enum { PISA_ROUTING_COV = 0, PISA_ROUTING_PLAIN = 1 };
/* PHASES = EXACT alone is keep-or-drop block-sparse attention; EXACT|ZEROTH omits H-bar.
 * FIRST needs ZEROTH (beta_t, the first-order weight, is the sum of the zeroth-order alpha_{t,j}):
 * the masks accepted are 1, 3 and 7; any other gives PISA_ERR_INVALID_ARGUMENT. */
enum { PISA_PHASE_EXACT = 1, PISA_PHASE_ZEROTH = 2, PISA_PHASE_FIRST = 4 };
/* First-order term of the unselected blocks. GLOBAL is the method: beta_t (q~_t H-bar), one
 * shared d x d matrix. BLOCK is the variant the method replaces (gist.science section 2 "Core
 * algorithm": per-block first-order terms would be memory-bound): sum_{j in U_i} alpha_{t,j}
 * (q~_t H_j) with every block's own H_j, stored as bf16 in the workspace (N_b d^2 * 2 bytes per
 * head) and streamed per query block. An ablation; bf16 only. */
enum { PISA_FIRST_ORDER_GLOBAL = 0, PISA_FIRST_ORDER_BLOCK = 1 };
/* The covariance-aware routing section of the gist.science summary writes M_j with a 2-norm
 * of a matrix. FROBENIUS reads it as ||.||_F (cheap, and an upper bound of the spectral norm);
 * SPECTRAL computes the largest singular value of H_j - H-bar (Lanczos on its Gram matrix, at
 * most 32 steps with full reorthogonalisation, then bisection on the tridiagonal: about 1e-6
 * relative for well-separated top singular values). Used by PISA_ROUTING_COV only. */
enum { PISA_NORM_FROBENIUS = 0, PISA_NORM_SPECTRAL = 1 };

typedef struct pisa_plan_info {
  int64_t L;
  int32_t H, d, B;
  int32_t n_blocks;     /* N_b = ceil(L / B) */
  int32_t k;            /* critical blocks per query block: clamp(ceil(keep N_b - 1e-9), 1, N_b) */
  int32_t n_last;       /* rows of the last block */
  int32_t dtype, routing, phases;
  double scale;
  size_t workspace_bytes;   /* device bytes pisa_plan_attach_workspace needs (256-B aligned) */
  double flops_stats;       /* 2 * 2 L d^2 per head: K^T V for H-bar and again for M_j */
  double flops_route;       /* 2 N_b^2 d per head */
  double flops_first;       /* per head: 2 L d^2 (q H-bar); BLOCK: (N_b - k) L (2 d^2 + 2 d) */
  double bytes_stats;       /* compulsory HBM bytes of the statistics kernels (reads Q,K,V,K,V) */
  int32_t first_order;      /* PISA_FIRST_ORDER_* */
  int32_t norm;             /* PISA_NORM_* */
} pisa_plan_info_t;

/* Create a plan for H heads of L tokens, head dim d, block size B, keeping a fraction `keep` of
 * the N_b key/value blocks per query block. The partition follows the AI Radio episode's paper
 * summary (queries, keys and values cut into blocks of size B; query block i keeps a critical set
 * S_i and approximates the rest, U_i); k = clamp(ceil(keep N_b - 1e-9), 1, N_b) blocks are kept.
 * Host only (no HIP call). *plan is set to NULL on error. Errors: INVALID_ARGUMENT for L, H, d or
 * B < 1, keep outside (0, 1] or a NULL plan pointer; UNSUPPORTED for sizes outside the list
 * above. */
pisa_status pisa_plan(int64_t L, int32_t H, int32_t d, int32_t B, double keep, pisa_plan_t **plan);

/* Set an option (see pisa_option). Changing the dtype, or selecting the block-wise first-order
 * variant, changes workspace_bytes: re-attach. */
pisa_status pisa_plan_set(pisa_plan_t *plan, pisa_option opt, double value);

/* Sizes, derived counts and the FLOP/byte model of the plan. */
pisa_status pisa_plan_info(const pisa_plan_t *plan, pisa_plan_info_t *info);

/* Attach caller-owned device memory of at least info.workspace_bytes, 256-byte aligned. The
 * plan keeps the pointer, not ownership. */
pisa_status pisa_plan_attach_workspace(pisa_plan_t *plan, void *dev_ptr, size_t bytes);

/* The whole forward pass: statistics, routing, fused piecewise attention, o_t = N_t / D_t for
 * every row (gist.science summary, section 2 "Core algorithm" for N_t, D_t and alpha; "Hardware
 * implementation" for the precompute and the three phases). Q, K, V: device [H, L, d] inputs,
 * read only; out: device [H, L, d], written in full. Enqueued on `stream` (asynchronous).
 * Equivalent to pisa_forward_stats + pisa_forward_route + pisa_forward_attend, with the argument
 * checks done once. It only launches kernels (no allocation, memset or synchronisation), so it
 * may be captured into a HIP graph; the captured graph keeps the pointers it was captured with.
 * Errors: INVALID_HANDLE, WORKSPACE, INVALID_ARGUMENT (see "Errors" above), DEVICE. */
pisa_status pisa_forward(pisa_plan_t *plan, const void *Q, const void *K, const void *V, void *out,
                         hipStream_t stream);

/* pisa_forward without an attached workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). The
 * statistics, selection and H-bar live in a static device array of 96 MiB per GPU (allocated
 * when the library's code is loaded, held until the process ends), which covers plans whose
 * workspace_bytes is at most 96 MiB (every bundled workload: the Wan2.1-14B-like 720p layer needs
 * 91 MiB); a larger plan gives PISA_ERR_WORKSPACE. The call allocates nothing and needs no
 * attached workspace (one attached to the plan is ignored). Every call on a GPU shares that GPU's
 * array and leaves its contents behind (every part is written before it is read, so nothing needs
 * clearing): calls that can overlap on one GPU (two streams, two threads) race and must be
 * serialised by the caller. Same arguments, checks and results as pisa_forward. */
pisa_status pisa_forward_noalloc(pisa_plan_t *plan, const void *Q, const void *K, const void *V, void *out,
                                 hipStream_t stream);

/* Stage 1: block statistics into the workspace (centroids, value sums, pooled queries, H-bar,
 * M_j). Reads Q, K, V. */
pisa_status pisa_forward_stats(pisa_plan_t *plan, const void *Q, const void *K, const void *V,
                               hipStream_t stream);

/* Stage 2: routing scores and per-query-block top-k into the workspace (needs stage 1). */
pisa_status pisa_forward_route(pisa_plan_t *plan, hipStream_t stream);

/* Stage 3: fused piecewise attention (needs stages 1 and 2 on the same inputs). */
pisa_status pisa_forward_attend(pisa_plan_t *plan, const void *Q, const void *K, const void *V,
                                void *out, hipStream_t stream);

/* Destroy a plan (does not free the attached workspace). Destroying NULL or twice returns
 * PISA_ERR_INVALID_HANDLE. */
pisa_status pisa_plan_destroy(pisa_plan_t *plan);

const char *pisa_status_string(pisa_status s);
const char *pisa_last_error(void);

/* Test support: copy statistics out of the workspace after a forward (async on `stream`, any
 * memory the HIP runtime can address; a NULL destination is skipped). Shapes (fp32):
 * qbar, kbar, vsum [H, N_b, d]; hbar [H, d, d]; M [H, N_b]. */
pisa_status pisa_debug_copy_stats(pisa_plan_t *plan, float *qbar, float *kbar, float *vsum,
                                  float *hbar, float *M, hipStream_t stream);

/* Test support: copy the selection: idx [H, N_b, k] int32, ascending block indices per row. */
pisa_status pisa_debug_copy_selection(pisa_plan_t *plan, int32_t *idx, hipStream_t stream);

/* Measurement support (no plan): `blocks` workgroups of 4 waves each run `iters` rounds of four
 * independent v_mfma_f32_32x32x16_bf16 on register operands, the instruction the attention
 * kernel is built on; FLOPs = blocks * 4 * 4 * iters * 32768. It gives the MFMA throughput and
 * shader clock the chip sustains under a pure MFMA load (the spec peak assumes 2.4 GHz).
 * out: device, blocks * 256 floats (results, kept live). clk: device, 2 * blocks uint64 per
 * workgroup: shader-clock ticks (s_memtime) and constant 100 MHz ticks (s_memrealtime) over the
 * loop. Asynchronous on `stream`. blocks in [1, 65536], iters in [1, 2^20], else
 * PISA_ERR_INVALID_ARGUMENT; a failed launch gives PISA_ERR_DEVICE. */
pisa_status pisa_debug_mfma_probe(int32_t blocks, int32_t iters, float *out, uint64_t *clk, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PISA_H_ */
