// libpisa C ABI: plans, workspace, stage dispatch, status reporting.
//
// The plan holds only host state (shapes and options); the caller owns all device memory.
// pisa_forward enqueues five launches on the caller's stream: block statistics pass, H-bar
// finalize, block covariance norms, routing, fused piecewise attention (plus the per-block
// first-order kernel when that variant is selected).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <unordered_set>

#include "../../include/pisa.h"
#include "pisa_internal.h"

namespace {

constexpr uint32_t kMagic = 0x50495341u;  // "PISA"
constexpr uint32_t kDead = 0xdeadbeefu;

thread_local char g_err[512] = "";

// Live plans: a destroyed or foreign handle is rejected without dereferencing it.
std::mutex g_plans_mu;
std::unordered_set<const void*>& live_plans() {
  static std::unordered_set<const void*> s;
  return s;
}

pisa_status fail(pisa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

struct pisa_plan_s {
  uint32_t magic;
  pisa::Dims dm;
  double keep;
  void* ws;
  size_t ws_bytes;
};

namespace pisa {

Layout workspace_layout(const Dims& dm) {
  Layout l{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const size_t H = dm.H, Nb = dm.Nb, d = dm.d;
  l.qbar = take(H * Nb * d * 4);
  l.kbar = take(H * Nb * d * 4);
  l.vsum = take(H * Nb * d * 4);
  const size_t slots = dm.dtype == PISA_DTYPE_BF16 ? (size_t)pisa::stat_slots(dm) : H * (size_t)dm.NC;
  l.G = take(slots * d * d * 4);
  l.hbar = take(H * d * d * 4);
  l.M = take(H * Nb * 4);
  if (dm.dtype == PISA_DTYPE_BF16) {
    l.kpart = take(slots * d * 4);
    l.kc = take(H * d * 4);
    l.kbar_lo = take(H * (size_t)dm.Nbp * d * 2);
    l.vbar_lo = take(H * (size_t)dm.Nbp * d * 2);
    l.hbarT_lo = take(H * d * d * 2);
  } else {
    l.kpart = l.kc = l.kbar_lo = l.vbar_lo = l.hbarT_lo = (size_t)-1;
  }
  l.idx = take(H * Nb * (size_t)dm.k * 4);
  if (pisa::block_first_order(dm)) {
    l.hjT_lo = take(H * Nb * d * d * 2);
    l.opart = take(H * (size_t)dm.L * d * 4);
    l.ml = take(H * (size_t)dm.L * 2 * 4);
  } else {
    l.hjT_lo = l.opart = l.ml = (size_t)-1;
  }
  l.total = off;
  return l;
}

Work workspace_pointers(const Dims& dm, void* base) {
  Layout l = workspace_layout(dm);
  char* b = static_cast<char*>(base);
  Work w{};
  w.qbar = reinterpret_cast<float*>(b + l.qbar);
  w.kbar = reinterpret_cast<float*>(b + l.kbar);
  w.vsum = reinterpret_cast<float*>(b + l.vsum);
  w.G = reinterpret_cast<float*>(b + l.G);
  w.hbar = reinterpret_cast<float*>(b + l.hbar);
  w.M = reinterpret_cast<float*>(b + l.M);
  if (dm.dtype == PISA_DTYPE_BF16) {
    w.kpart = reinterpret_cast<float*>(b + l.kpart);
    w.kc = reinterpret_cast<float*>(b + l.kc);
    w.kbar_lo = b + l.kbar_lo;
    w.vbar_lo = b + l.vbar_lo;
    w.hbarT_lo = b + l.hbarT_lo;
  }
  w.idx = reinterpret_cast<int32_t*>(b + l.idx);
  if (block_first_order(dm)) {
    w.hjT_lo = b + l.hjT_lo;
    w.opart = reinterpret_cast<float*>(b + l.opart);
    w.ml = reinterpret_cast<float*>(b + l.ml);
  }
  return w;
}

}  // namespace pisa

namespace {

bool valid_plan(const pisa_plan_t* p) {
  if (p == nullptr) return false;
  std::lock_guard<std::mutex> g(g_plans_mu);
  return live_plans().count(p) != 0 && p->magic == kMagic;
}

pisa_status check_supported(const pisa::Dims& dm) {
  if (dm.dtype == PISA_DTYPE_BF16 && dm.d != 128)
    return fail(PISA_ERR_UNSUPPORTED, "bf16 path supports d = 128 only (got d = %d)", dm.d);
  if (dm.d != 64 && dm.d != 128) return fail(PISA_ERR_UNSUPPORTED, "d must be 64 or 128 (got %d)", dm.d);
  if (dm.B != 64 && dm.B != 128) return fail(PISA_ERR_UNSUPPORTED, "B must be 64 or 128 (got %d)", dm.B);
  if (dm.Nb > 8192) return fail(PISA_ERR_UNSUPPORTED, "at most 8192 blocks per head (got %d)", dm.Nb);
  if (dm.first_block && dm.dtype != PISA_DTYPE_BF16)
    return fail(PISA_ERR_UNSUPPORTED, "the block-wise first-order variant is implemented for bf16 only");
  return PISA_OK;
}

void derive(pisa::Dims& dm, double keep) {
  dm.Nb = (int)((dm.L + dm.B - 1) / dm.B);
  dm.n_last = dm.L - (dm.Nb - 1) * dm.B;
  double kk = ceil(keep * dm.Nb - 1e-9);
  if (kk < 1) kk = 1;
  if (kk > dm.Nb) kk = dm.Nb;
  dm.k = (int)kk;
  // fp32 statistics workgroups: chunks of 16 blocks, halved (down to 1) while there are fewer
  // than 512 workgroups (two per CU), so that small layers still spread over the chip
  dm.chunk = pisa::kStatsChunk;
  while (dm.chunk > 1 && (long long)((dm.Nb + dm.chunk - 1) / dm.chunk) * dm.H < 512) dm.chunk /= 2;
  dm.NC = (dm.Nb + dm.chunk - 1) / dm.chunk;
  // bf16 statistics passes: one range of (head, block) pairs per workgroup, two workgroups per CU
  // on a 256-CU chip, and at least about 4 blocks per range so that each partial sum written
  // (64 KB) stands for several blocks
  const long long pairs = (long long)dm.H * dm.Nb;
  dm.SW = (int)std::min<long long>(pisa::kStatsWorkgroups, std::max<long long>(1, (pairs + 3) / 4));
  dm.Nbp = ((dm.Nb + dm.B - 1) / dm.B) * dm.B;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

pisa_status check_device() {
  int n = 0;
  hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess || n <= 0)
    return fail(PISA_ERR_DEVICE, "no HIP device available (%s)", hipGetErrorString(e));
  return PISA_OK;
}

// `bytes` from ptr must be device memory of one allocation. A host address, or a range that runs
// past the end of its allocation, would fault the kernels; it is rejected here instead. A failed
// query leaves no error behind for the launch checks that follow (hipGetLastError clears it).
pisa_status check_device_memory(const void* ptr, size_t bytes, const char* name) {
  hipPointerAttribute_t a{};
  hipError_t e = hipPointerGetAttributes(&a, ptr);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(PISA_ERR_INVALID_ARGUMENT, "%s (%p) is not device memory (%s)", name, ptr, hipGetErrorString(e));
  }
  if (a.type != hipMemoryTypeDevice && a.type != hipMemoryTypeManaged)
    return fail(PISA_ERR_INVALID_ARGUMENT, "%s (%p) is not device memory (memory type %d)", name, ptr, (int)a.type);
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  e = hipMemGetAddressRange(&base, &size, const_cast<void*>(ptr));
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return PISA_OK;  // the range query is not available for every allocation kind
  }
  const size_t left = size - (size_t)(static_cast<const char*>(ptr) - static_cast<const char*>(base));
  if (bytes > left)
    return fail(PISA_ERR_INVALID_ARGUMENT, "%s: %zu bytes needed from %p, but its allocation ends after %zu",
                name, bytes, ptr, left);
  return PISA_OK;
}

pisa_status check_ready(pisa_plan_t* p) {
  if (!valid_plan(p)) return fail(PISA_ERR_INVALID_HANDLE, "invalid or destroyed plan");
  if (p->ws == nullptr) return fail(PISA_ERR_WORKSPACE, "no workspace attached");
  pisa_status s = check_supported(p->dm);
  if (s != PISA_OK) return s;
  size_t need = pisa::workspace_layout(p->dm).total;
  if (p->ws_bytes < need)
    return fail(PISA_ERR_WORKSPACE, "workspace too small: %zu bytes attached, %zu needed", p->ws_bytes, need);
  return PISA_OK;
}

pisa_status check_tensors(const pisa_plan_t* p, const void* Q, const void* K, const void* V,
                          const void* out) {
  const void* ptrs[4] = {Q, K, V, out};
  const char* names[4] = {"Q", "K", "V", "out"};
  for (int i = 0; i < 4; ++i) {
    if (i == 3 && out == nullptr) continue;  // stages that do not write out
    if (ptrs[i] == nullptr) return fail(PISA_ERR_INVALID_ARGUMENT, "%s is NULL", names[i]);
    if (!aligned16(ptrs[i])) return fail(PISA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", names[i]);
  }
  if (out != nullptr) {
    size_t esz = p->dm.dtype == PISA_DTYPE_BF16 ? 2 : 4;
    size_t bytes = (size_t)p->dm.H * p->dm.L * p->dm.d * esz;
    uintptr_t o0 = (uintptr_t)out, o1 = o0 + bytes;
    for (int i = 0; i < 3; ++i) {
      uintptr_t a0 = (uintptr_t)ptrs[i], a1 = a0 + bytes;
      if (a0 < o1 && o0 < a1) return fail(PISA_ERR_INVALID_ARGUMENT, "out overlaps %s", names[i]);
    }
  }
  return PISA_OK;
}

// PISA_DEBUG_SYNC set in the environment: synchronise after every launch and report the kernel
// that failed (read once per process).
bool debug_sync() {
  static const bool on = getenv("PISA_DEBUG_SYNC") != nullptr;
  return on;
}

pisa_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(PISA_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
  if (debug_sync()) {
    e = hipDeviceSynchronize();
    if (e != hipSuccess) return fail(PISA_ERR_DEVICE, "%s (synchronised): %s", what, hipGetErrorString(e));
  }
  return PISA_OK;
}

pisa_status check_inputs_resident(const pisa_plan_t* p, const void* Q, const void* K, const void* V,
                                  const void* out);

// What a call reads and writes besides the workspace.
enum Uses { kWorkspaceOnly, kInputs, kInputsAndOut };

// Every check of a call that touches device memory, once per call: plan, workspace, pointer
// arguments (NULL, alignment, overlap), device present, and each buffer resident in device memory
// with room for its extent.
pisa_status prepare(pisa_plan_t* p, const void* Q, const void* K, const void* V, const void* out, Uses uses) {
  pisa_status s = check_ready(p);
  if (s != PISA_OK) return s;
  if (uses == kInputsAndOut && out == nullptr) return fail(PISA_ERR_INVALID_ARGUMENT, "out is NULL");
  const bool tensors = uses != kWorkspaceOnly;
  if (tensors && (s = check_tensors(p, Q, K, V, out)) != PISA_OK) return s;
  if ((s = check_device()) != PISA_OK) return s;
  if ((s = check_device_memory(p->ws, pisa::workspace_layout(p->dm).total, "workspace")) != PISA_OK) return s;
  return tensors ? check_inputs_resident(p, Q, K, V, out) : PISA_OK;
}

// Q, K, V (and out, when given) in device memory with room for [H, L, d] each.
pisa_status check_inputs_resident(const pisa_plan_t* p, const void* Q, const void* K, const void* V,
                                  const void* out) {
  const pisa::Dims& dm = p->dm;
  pisa_status s;
  const size_t bytes = (size_t)dm.H * dm.L * dm.d * (dm.dtype == PISA_DTYPE_BF16 ? 2 : 4);
  const void* ptrs[4] = {Q, K, V, out};
  const char* names[4] = {"Q", "K", "V", "out"};
  for (int i = 0; i < 4; ++i)
    if (ptrs[i] != nullptr && (s = check_device_memory(ptrs[i], bytes, names[i])) != PISA_OK) return s;
  return PISA_OK;
}

// The stages' launches, on a plan and arguments that prepare() accepted.
pisa_status run_stats(pisa_plan_t* p, void* ws, const void* Q, const void* K, const void* V, hipStream_t stream) {
  pisa::Work w = pisa::workspace_pointers(p->dm, ws);
  pisa_status s;
  if ((s = launched(pisa::launch_stats_pass(p->dm, w, Q, K, V, stream), "stats pass")) != PISA_OK) return s;
  if ((s = launched(pisa::launch_stats_finalize(p->dm, w, stream), "H-bar finalize")) != PISA_OK) return s;
  if (p->dm.routing == PISA_ROUTING_COV || pisa::block_first_order(p->dm))
    return launched(pisa::launch_stats_cov(p->dm, w, K, V, stream), "block covariance norms");
  return PISA_OK;
}

pisa_status run_route(pisa_plan_t* p, void* ws, hipStream_t stream) {
  pisa::Work w = pisa::workspace_pointers(p->dm, ws);
  return launched(pisa::launch_route(p->dm, w, stream), "route");
}

pisa_status run_attend(pisa_plan_t* p, void* ws, const void* Q, const void* K, const void* V, void* out,
                       hipStream_t stream) {
  pisa::Work w = pisa::workspace_pointers(p->dm, ws);
  pisa_status s;
  if ((s = launched(pisa::launch_attend(p->dm, w, Q, K, V, out, stream), "attend")) != PISA_OK) return s;
  if (pisa::block_first_order(p->dm))
    return launched(pisa::launch_first_block_bf16(p->dm, w, Q, out, stream), "block first order");
  return PISA_OK;
}

pisa_status run_forward(pisa_plan_t* p, void* ws, const void* Q, const void* K, const void* V, void* out,
                        hipStream_t stream) {
  pisa_status s;
  if ((s = run_stats(p, ws, Q, K, V, stream)) != PISA_OK) return s;
  if ((s = run_route(p, ws, stream)) != PISA_OK) return s;
  return run_attend(p, ws, Q, K, V, out, stream);
}

}  // namespace

extern "C" {

pisa_status pisa_plan(int64_t L, int32_t H, int32_t d, int32_t B, double keep, pisa_plan_t** plan) {
  if (plan == nullptr) return fail(PISA_ERR_INVALID_ARGUMENT, "plan output pointer is NULL");
  *plan = nullptr;
  if (L < 1 || H < 1 || d < 1 || B < 1)
    return fail(PISA_ERR_INVALID_ARGUMENT, "L, H, d, B must be >= 1 (got %lld, %d, %d, %d)", (long long)L, H, d, B);
  if (!(keep > 0.0 && keep <= 1.0)) return fail(PISA_ERR_INVALID_ARGUMENT, "keep must be in (0, 1] (got %g)", keep);
  if ((double)H * (double)L * (double)d >= 2147483648.0)
    return fail(PISA_ERR_UNSUPPORTED, "H * L * d must be < 2^31 elements");
  pisa::Dims dm{};
  dm.H = H;
  dm.L = (int)L;
  dm.d = d;
  dm.B = B;
  dm.scale = (float)(1.0 / sqrt((double)d));
  dm.routing = PISA_ROUTING_COV;
  dm.phases = PISA_PHASE_EXACT | PISA_PHASE_ZEROTH | PISA_PHASE_FIRST;
  dm.dtype = d == 128 ? PISA_DTYPE_BF16 : PISA_DTYPE_F32;
  derive(dm, keep);
  pisa_status s = check_supported(dm);
  if (s != PISA_OK) return s;
  pisa_plan_t* p = new (std::nothrow) pisa_plan_s();
  if (p == nullptr) return fail(PISA_ERR_INVALID_ARGUMENT, "out of host memory");
  p->magic = kMagic;
  p->dm = dm;
  p->keep = keep;
  p->ws = nullptr;
  p->ws_bytes = 0;
  {
    std::lock_guard<std::mutex> g(g_plans_mu);
    live_plans().insert(p);
  }
  *plan = p;
  return PISA_OK;
}

pisa_status pisa_plan_set(pisa_plan_t* p, pisa_option opt, double value) {
  if (!valid_plan(p)) return fail(PISA_ERR_INVALID_HANDLE, "invalid or destroyed plan");
  pisa::Dims dm = p->dm;
  switch (opt) {
    case PISA_OPT_DTYPE:
      if (value != PISA_DTYPE_BF16 && value != PISA_DTYPE_F32)
        return fail(PISA_ERR_INVALID_ARGUMENT, "dtype must be PISA_DTYPE_BF16 or PISA_DTYPE_F32");
      dm.dtype = (int)value;
      break;
    case PISA_OPT_SCALE:
      if (!(value > 0.0) || !isfinite(value)) return fail(PISA_ERR_INVALID_ARGUMENT, "scale must be finite and > 0");
      dm.scale = (float)value;
      break;
    case PISA_OPT_ROUTING:
      if (value != PISA_ROUTING_COV && value != PISA_ROUTING_PLAIN)
        return fail(PISA_ERR_INVALID_ARGUMENT, "routing must be PISA_ROUTING_COV or PISA_ROUTING_PLAIN");
      dm.routing = (int)value;
      break;
    case PISA_OPT_PHASES: {
      int m = (int)value;
      if ((double)m != value || m < 1 || m > 7 || !(m & PISA_PHASE_EXACT))
        return fail(PISA_ERR_INVALID_ARGUMENT, "phases must be a mask of PISA_PHASE_* including EXACT");
      // beta_t, the weight of the first-order term, is the sum of the zeroth-order alpha_{t,j}:
      // there is no first-order term without the zeroth-order one
      if ((m & PISA_PHASE_FIRST) && !(m & PISA_PHASE_ZEROTH))
        return fail(PISA_ERR_INVALID_ARGUMENT, "PISA_PHASE_FIRST needs PISA_PHASE_ZEROTH");
      dm.phases = m;
      break;
    }
    case PISA_OPT_NORM:
      if (value != PISA_NORM_FROBENIUS && value != PISA_NORM_SPECTRAL)
        return fail(PISA_ERR_INVALID_ARGUMENT, "norm must be PISA_NORM_FROBENIUS or PISA_NORM_SPECTRAL");
      dm.spectral = (int)value;
      break;
    case PISA_OPT_FIRST_ORDER:
      if (value != PISA_FIRST_ORDER_GLOBAL && value != PISA_FIRST_ORDER_BLOCK)
        return fail(PISA_ERR_INVALID_ARGUMENT, "first order must be PISA_FIRST_ORDER_GLOBAL or PISA_FIRST_ORDER_BLOCK");
      dm.first_block = (int)value;
      break;
    default:
      return fail(PISA_ERR_INVALID_ARGUMENT, "unknown option %d", (int)opt);
  }
  pisa_status s = check_supported(dm);
  if (s != PISA_OK) return s;
  p->dm = dm;
  return PISA_OK;
}

pisa_status pisa_plan_info(const pisa_plan_t* p, pisa_plan_info_t* info) {
  if (!valid_plan(p)) return fail(PISA_ERR_INVALID_HANDLE, "invalid or destroyed plan");
  if (info == nullptr) return fail(PISA_ERR_INVALID_ARGUMENT, "info is NULL");
  const pisa::Dims& dm = p->dm;
  memset(info, 0, sizeof(*info));
  info->L = dm.L;
  info->H = dm.H;
  info->d = dm.d;
  info->B = dm.B;
  info->n_blocks = dm.Nb;
  info->k = dm.k;
  info->n_last = dm.n_last;
  info->dtype = dm.dtype;
  info->routing = dm.routing;
  info->phases = dm.phases;
  info->scale = dm.scale;
  info->workspace_bytes = pisa::workspace_layout(dm).total;
  double H = dm.H, L = dm.L, d = dm.d, Nb = dm.Nb;
  double e = dm.dtype == PISA_DTYPE_BF16 ? 2.0 : 4.0;
  info->flops_stats = H * 2.0 * (2.0 * L * d * d);
  info->flops_route = H * 2.0 * Nb * Nb * d;
  const bool tail = dm.k < dm.Nb && (dm.phases & PISA_PHASE_ZEROTH) && (dm.phases & PISA_PHASE_FIRST);
  info->flops_first = !tail ? 0.0
                      : dm.first_block ? H * (Nb - dm.k) * L * (2.0 * d * d + 2.0 * d)
                                       : H * 2.0 * L * d * d;
  info->bytes_stats = H * 5.0 * L * d * e;
  info->first_order = dm.first_block;
  info->norm = dm.spectral;
  return PISA_OK;
}

pisa_status pisa_plan_attach_workspace(pisa_plan_t* p, void* dev_ptr, size_t bytes) {
  if (!valid_plan(p)) return fail(PISA_ERR_INVALID_HANDLE, "invalid or destroyed plan");
  if (dev_ptr == nullptr) return fail(PISA_ERR_WORKSPACE, "workspace pointer is NULL");
  if ((reinterpret_cast<uintptr_t>(dev_ptr) & 255u) != 0) return fail(PISA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  size_t need = pisa::workspace_layout(p->dm).total;
  if (bytes < need) return fail(PISA_ERR_WORKSPACE, "workspace too small: %zu bytes given, %zu needed", bytes, need);
  p->ws = dev_ptr;
  p->ws_bytes = bytes;
  return PISA_OK;
}

pisa_status pisa_forward_stats(pisa_plan_t* p, const void* Q, const void* K, const void* V, hipStream_t stream) {
  pisa_status s = prepare(p, Q, K, V, nullptr, kInputs);
  return s != PISA_OK ? s : run_stats(p, p->ws, Q, K, V, stream);
}

pisa_status pisa_forward_route(pisa_plan_t* p, hipStream_t stream) {
  pisa_status s = prepare(p, nullptr, nullptr, nullptr, nullptr, kWorkspaceOnly);
  return s != PISA_OK ? s : run_route(p, p->ws, stream);
}

pisa_status pisa_forward_attend(pisa_plan_t* p, const void* Q, const void* K, const void* V, void* out,
                                hipStream_t stream) {
  pisa_status s = prepare(p, Q, K, V, out, kInputsAndOut);
  return s != PISA_OK ? s : run_attend(p, p->ws, Q, K, V, out, stream);
}

pisa_status pisa_forward(pisa_plan_t* p, const void* Q, const void* K, const void* V, void* out, hipStream_t stream) {
  pisa_status s = prepare(p, Q, K, V, out, kInputsAndOut);
  if (s != PISA_OK) return s;
  return run_forward(p, p->ws, Q, K, V, out, stream);
}

pisa_status pisa_forward_noalloc(pisa_plan_t* p, const void* Q, const void* K, const void* V, void* out,
                                 hipStream_t stream) {
  if (!valid_plan(p)) return fail(PISA_ERR_INVALID_HANDLE, "invalid or destroyed plan");
  pisa_status s = check_supported(p->dm);
  if (s != PISA_OK) return s;
  const size_t need = pisa::workspace_layout(p->dm).total;
  if (need > pisa::kStaticWorkspaceBytes)
    return fail(PISA_ERR_WORKSPACE, "the plan needs %zu bytes of workspace; the static workspace holds %zu",
                need, pisa::kStaticWorkspaceBytes);
  if (out == nullptr) return fail(PISA_ERR_INVALID_ARGUMENT, "out is NULL");
  if ((s = check_tensors(p, Q, K, V, out)) != PISA_OK) return s;
  if ((s = check_device()) != PISA_OK) return s;
  if ((s = check_inputs_resident(p, Q, K, V, out)) != PISA_OK) return s;
  void* ws = nullptr;
  hipError_t e = pisa::static_workspace(stream, &ws);
  if (e != hipSuccess) return fail(PISA_ERR_DEVICE, "static workspace lookup: %s", hipGetErrorString(e));
  return run_forward(p, ws, Q, K, V, out, stream);
}

pisa_status pisa_plan_destroy(pisa_plan_t* p) {
  {
    std::lock_guard<std::mutex> g(g_plans_mu);
    if (p == nullptr || live_plans().erase(p) == 0)
      return fail(PISA_ERR_INVALID_HANDLE, "invalid or destroyed plan");
  }
  p->magic = kDead;
  delete p;
  return PISA_OK;
}

const char* pisa_status_string(pisa_status s) {
  switch (s) {
    case PISA_OK: return "PISA_OK";
    case PISA_ERR_INVALID_ARGUMENT: return "PISA_ERR_INVALID_ARGUMENT";
    case PISA_ERR_UNSUPPORTED: return "PISA_ERR_UNSUPPORTED";
    case PISA_ERR_INVALID_HANDLE: return "PISA_ERR_INVALID_HANDLE";
    case PISA_ERR_WORKSPACE: return "PISA_ERR_WORKSPACE";
    case PISA_ERR_DEVICE: return "PISA_ERR_DEVICE";
  }
  return "PISA_ERR_UNKNOWN";
}

const char* pisa_last_error(void) { return g_err; }

pisa_status pisa_debug_copy_stats(pisa_plan_t* p, float* qbar, float* kbar, float* vsum, float* hbar, float* M,
                                  hipStream_t stream) {
  pisa_status s = check_ready(p);
  if (s != PISA_OK) return s;
  if ((s = check_device()) != PISA_OK) return s;
  const pisa::Dims& dm = p->dm;
  pisa::Work w = pisa::workspace_pointers(dm, p->ws);
  size_t nbd = (size_t)dm.H * dm.Nb * dm.d * 4;
  struct {
    void* dst;
    const void* src;
    size_t bytes;
  } cp[5] = {{qbar, w.qbar, nbd}, {kbar, w.kbar, nbd}, {vsum, w.vsum, nbd},
             {hbar, w.hbar, (size_t)dm.H * dm.d * dm.d * 4}, {M, w.M, (size_t)dm.H * dm.Nb * 4}};
  for (auto& c : cp) {
    if (c.dst == nullptr) continue;
    hipError_t e = hipMemcpyAsync(c.dst, c.src, c.bytes, hipMemcpyDefault, stream);
    if (e != hipSuccess) return fail(PISA_ERR_DEVICE, "debug copy: %s", hipGetErrorString(e));
  }
  return PISA_OK;
}

pisa_status pisa_debug_copy_selection(pisa_plan_t* p, int32_t* idx, hipStream_t stream) {
  pisa_status s = check_ready(p);
  if (s != PISA_OK) return s;
  if (idx == nullptr) return fail(PISA_ERR_INVALID_ARGUMENT, "idx is NULL");
  if ((s = check_device()) != PISA_OK) return s;
  const pisa::Dims& dm = p->dm;
  pisa::Work w = pisa::workspace_pointers(dm, p->ws);
  hipError_t e = hipMemcpyAsync(idx, w.idx, (size_t)dm.H * dm.Nb * dm.k * 4, hipMemcpyDefault, stream);
  if (e != hipSuccess) return fail(PISA_ERR_DEVICE, "debug copy: %s", hipGetErrorString(e));
  return PISA_OK;
}

pisa_status pisa_debug_mfma_probe(int32_t blocks, int32_t iters, float* out, uint64_t* clk, hipStream_t stream) {
  if (blocks < 1 || blocks > 65536) return fail(PISA_ERR_INVALID_ARGUMENT, "blocks must be in [1, 65536], got %d", blocks);
  if (iters < 1 || iters > (1 << 20)) return fail(PISA_ERR_INVALID_ARGUMENT, "iters must be in [1, 2^20], got %d", iters);
  if (out == nullptr || clk == nullptr) return fail(PISA_ERR_INVALID_ARGUMENT, "out and clk must not be NULL");
  pisa_status s = check_device();
  if (s != PISA_OK) return s;
  return launched(pisa::launch_mfma_probe(blocks, iters, out, clk, stream), "mfma probe");
}

}  // extern "C"

namespace pisa {

hipError_t launch_stats_pass(const Dims& dm, const Work& w, const void* Q, const void* K, const void* V,
                             hipStream_t s) {
  return dm.dtype == PISA_DTYPE_BF16 ? launch_stats_pass_bf16(dm, w, Q, K, V, s)
                                     : launch_stats_pass_f32(dm, w, Q, K, V, s);
}

hipError_t launch_stats_cov(const Dims& dm, const Work& w, const void* K, const void* V, hipStream_t s) {
  return dm.dtype == PISA_DTYPE_BF16 ? launch_stats_cov_bf16(dm, w, K, V, s) : launch_stats_cov_f32(dm, w, K, V, s);
}

hipError_t launch_attend(const Dims& dm, const Work& w, const void* Q, const void* K, const void* V, void* out,
                         hipStream_t s) {
  return dm.dtype == PISA_DTYPE_BF16 ? launch_attend_bf16(dm, w, Q, K, V, out, s)
                                     : launch_attend_f32(dm, w, Q, K, V, out, s);
}

}  // namespace pisa
