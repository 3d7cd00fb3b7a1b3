"""ctypes binding of libpisa (include/pisa.h). Argument marshalling only: every step of the
forward pass runs in the library's HIP kernels. If libpisa.so has not been built, loading raises;
there is no fallback implementation."""

from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpisa.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "pisa.h")

PISA_OK = 0
STATUS = {0: "PISA_OK", 1: "PISA_ERR_INVALID_ARGUMENT", 2: "PISA_ERR_UNSUPPORTED",
          3: "PISA_ERR_INVALID_HANDLE", 4: "PISA_ERR_WORKSPACE", 5: "PISA_ERR_DEVICE"}
DTYPE_BF16, DTYPE_F32 = 0, 1
ROUTING_COV, ROUTING_PLAIN = 0, 1
PHASE_EXACT, PHASE_ZEROTH, PHASE_FIRST = 1, 2, 4
FIRST_ORDER_GLOBAL, FIRST_ORDER_BLOCK = 0, 1
NORM_FROBENIUS, NORM_SPECTRAL = 0, 1
OPT_DTYPE, OPT_SCALE, OPT_ROUTING, OPT_PHASES, OPT_FIRST_ORDER, OPT_NORM = 0, 1, 2, 3, 4, 5


class PisaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {STATUS.get(status, status)}: {detail}")
        self.status = status


class PlanInfo(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int64), ("H", ctypes.c_int32), ("d", ctypes.c_int32),
                ("B", ctypes.c_int32), ("n_blocks", ctypes.c_int32), ("k", ctypes.c_int32),
                ("n_last", ctypes.c_int32), ("dtype", ctypes.c_int32), ("routing", ctypes.c_int32),
                ("phases", ctypes.c_int32), ("scale", ctypes.c_double),
                ("workspace_bytes", ctypes.c_size_t), ("flops_stats", ctypes.c_double),
                ("flops_route", ctypes.c_double), ("flops_first", ctypes.c_double),
                ("bytes_stats", ctypes.c_double), ("first_order", ctypes.c_int32), ("norm", ctypes.c_int32)]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f, _ in self._fields_}


_P = ctypes.c_void_p
_SIGS = {
    "pisa_plan": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                 ctypes.c_double, ctypes.POINTER(_P)]),
    "pisa_plan_set": (ctypes.c_int, [_P, ctypes.c_int, ctypes.c_double]),
    "pisa_plan_info": (ctypes.c_int, [_P, ctypes.POINTER(PlanInfo)]),
    "pisa_plan_attach_workspace": (ctypes.c_int, [_P, _P, ctypes.c_size_t]),
    "pisa_forward": (ctypes.c_int, [_P, _P, _P, _P, _P, _P]),
    "pisa_forward_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P]),
    "pisa_forward_stats": (ctypes.c_int, [_P, _P, _P, _P, _P]),
    "pisa_forward_route": (ctypes.c_int, [_P, _P]),
    "pisa_forward_attend": (ctypes.c_int, [_P, _P, _P, _P, _P, _P]),
    "pisa_plan_destroy": (ctypes.c_int, [_P]),
    "pisa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pisa_last_error": (ctypes.c_char_p, []),
    "pisa_debug_copy_stats": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P]),
    "pisa_debug_copy_selection": (ctypes.c_int, [_P, _P, _P]),
    "pisa_debug_mfma_probe": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, _P, _P, _P]),
}

_lib = None


def header_functions(path: str = HEADER):
    """Names of the functions include/pisa.h declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pisa_[a-z_]+)\s*\(", text)))


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    # torch-ROCm ships its own HIP runtime under the same soname: load torch first so that libpisa
    # binds to the runtime that owns torch's device memory and streams (one runtime per process)
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(path):
        raise RuntimeError(f"libpisa is not built ({path} missing): run "
                           "`python -m sparse_attention_diffusion_pool_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def last_error() -> str:
    return load().pisa_last_error().decode(errors="replace")


def check(status: int, where: str) -> None:
    if status != PISA_OK:
        raise PisaError(status, where, last_error())


def _ptr(t) -> int:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _tensor_ptr(t, name: str, info: dict) -> int:
    """Address of a Q/K/V/out argument. A torch tensor must have the plan's dtype, shape [H, L, d],
    be contiguous and live on the GPU; anything else raises here, before the library is called (a
    transposed [L, H, d] -> [H, L, d] view would otherwise be read with the wrong strides, and a host
    tensor's address would reach the kernels). Raw integer addresses are passed through: the library
    checks that they point into device memory large enough for the tensor."""
    if t is None or isinstance(t, int):
        return t
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor or a device address, got {type(t).__name__}")
    want = torch.bfloat16 if info["dtype"] == DTYPE_BF16 else torch.float32
    if t.dtype != want:
        raise TypeError(f"{name}: dtype {t.dtype}, the plan computes in {want}")
    shape = (info["H"], info["L"], info["d"])
    if tuple(t.shape) != shape:
        raise ValueError(f"{name}: shape {tuple(t.shape)}, the plan expects [H, L, d] = {list(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: not contiguous (strides {t.stride()}); a transposed view needs "
                         ".contiguous() first")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: on {t.device}, the library reads device memory")
    return t.data_ptr()


class Plan:
    """A libpisa plan. Tensors are passed as torch tensors (device memory, the plan's dtype, shape
    [H, L, d], contiguous; checked before the call) or raw device addresses."""

    def __init__(self, L: int, H: int, d: int, B: int, keep: float, dtype=None, scale=None,
                 routing=None, phases=None, first_order=None, norm=None):
        lib = load()
        h = _P()
        check(lib.pisa_plan(int(L), int(H), int(d), int(B), float(keep), ctypes.byref(h)), "pisa_plan")
        self._h = h
        self._ws = None
        for opt, val in ((OPT_DTYPE, dtype), (OPT_SCALE, scale), (OPT_ROUTING, routing),
                         (OPT_PHASES, phases), (OPT_FIRST_ORDER, first_order), (OPT_NORM, norm)):
            if val is not None:
                check(lib.pisa_plan_set(self._h, opt, float(val)), "pisa_plan_set")

    @property
    def handle(self):
        return self._h

    def info(self) -> dict:
        inf = PlanInfo()
        check(load().pisa_plan_info(self._h, ctypes.byref(inf)), "pisa_plan_info")
        return inf.as_dict()

    def attach_workspace(self, ws=None, device="cuda"):
        """Attach caller memory, or allocate a torch uint8 buffer of the needed size."""
        if ws is None:
            import torch
            ws = torch.empty(self.info()["workspace_bytes"] + 256, dtype=torch.uint8, device=device)
            off = (-ws.data_ptr()) % 256
            ws = ws[off:]
        check(load().pisa_plan_attach_workspace(self._h, _ptr(ws), ws.numel()), "pisa_plan_attach_workspace")
        self._ws = ws
        return ws

    def _args(self, **tensors):
        info = self.info()
        return [_tensor_ptr(t, name, info) for name, t in tensors.items()]

    def forward(self, Q, K, V, out, stream=None):
        q, k, v, o = self._args(Q=Q, K=K, V=V, out=out)
        check(load().pisa_forward(self._h, q, k, v, o, _stream(stream)), "pisa_forward")
        return out

    def forward_noalloc(self, Q, K, V, out, stream=None):
        """pisa_forward_noalloc: the forward pass on the library's static per-GPU workspace."""
        q, k, v, o = self._args(Q=Q, K=K, V=V, out=out)
        check(load().pisa_forward_noalloc(self._h, q, k, v, o, _stream(stream)), "pisa_forward_noalloc")
        return out

    def forward_stats(self, Q, K, V, stream=None):
        q, k, v = self._args(Q=Q, K=K, V=V)
        check(load().pisa_forward_stats(self._h, q, k, v, _stream(stream)), "pisa_forward_stats")

    def forward_route(self, stream=None):
        check(load().pisa_forward_route(self._h, _stream(stream)), "pisa_forward_route")

    def forward_attend(self, Q, K, V, out, stream=None):
        q, k, v, o = self._args(Q=Q, K=K, V=V, out=out)
        check(load().pisa_forward_attend(self._h, q, k, v, o, _stream(stream)), "pisa_forward_attend")
        return out

    def debug_copy_stats(self, qbar=None, kbar=None, vsum=None, hbar=None, M=None, stream=None):
        check(load().pisa_debug_copy_stats(self._h, _ptr(qbar), _ptr(kbar), _ptr(vsum), _ptr(hbar), _ptr(M),
                                           _stream(stream)), "pisa_debug_copy_stats")

    def debug_copy_selection(self, idx, stream=None):
        check(load().pisa_debug_copy_selection(self._h, _ptr(idx), _stream(stream)), "pisa_debug_copy_selection")

    def destroy(self):
        if self._h is not None and self._h.value is not None:
            check(load().pisa_plan_destroy(self._h), "pisa_plan_destroy")
        self._h = None

    def __del__(self):
        try:
            if getattr(self, "_h", None) is not None and self._h.value is not None:
                load().pisa_plan_destroy(self._h)
        except Exception:
            pass


def pisa_attention(Q, K, V, B: int, keep: float, routing=None, phases=None, scale=None, stream=None):
    """Convenience: out = PISA(Q, K, V) for device tensors [H, L, d] (bf16 or fp32)."""
    import torch
    H, L, d = Q.shape
    dtype = DTYPE_BF16 if Q.dtype == torch.bfloat16 else DTYPE_F32
    plan = Plan(L, H, d, B, keep, dtype=dtype, routing=routing, phases=phases, scale=scale)
    plan.attach_workspace(device=Q.device)
    out = torch.empty_like(Q)
    plan.forward(Q, K, V, out, stream)
    return out, plan


def mfma_probe(out, clk, blocks: int, iters: int, stream=None) -> None:
    """pisa_debug_mfma_probe: out float32 [blocks * 256], clk int64 [blocks * 2] (device tensors)."""
    check(load().pisa_debug_mfma_probe(int(blocks), int(iters), _ptr(out), _ptr(clk), _stream(stream)),
          "pisa_debug_mfma_probe")
