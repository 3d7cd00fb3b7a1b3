"""Seeded synthetic Q/K/V for diffusion-transformer self-attention layers.

The method's pages evaluate on pretrained video and image DiTs (Wan2.1, HunyuanVideo, FLUX.1);
their weights and activations are not available here, so these generators stand in for them with
the same token counts, head counts, head dim and block size, and with the structure that makes
blocks of neighbouring tokens similar: every image/video token carries random Fourier features
of its normalised grid coordinate, projected to Q and K by per-head Gaussian matrices, plus
isotropic noise. Text tokens (FLUX-like, Hunyuan-like layers) follow the grid tokens and carry
i.i.d. N(0,1) features. V is i.i.d. N(0,1) everywhere.

Recipe (one numpy ``SeedSequence(1000 + cfg_id)`` per workload, spawned into ``2 + H`` children):

* child 0: ``Omega ~ N(0, (2 pi)^2)`` of shape ``[D, ndim]`` and ``b ~ U[0, 2 pi)`` of shape ``[D]``,
  shared by Q, K and every head; ``phi(x) = sqrt(2/D) cos(Omega x + b)`` with ``x`` the token's
  grid coordinate normalised per axis to ``[0, 1]`` (raster order, first axis slowest).
* child 1: reserved (unused) so that adding global draws later does not shift head streams.
* child 2 + h (head h), drawn in this order: ``W_Q, W_K ~ N(0,1)^{D x d}``, ``eps_Q, eps_K ~
  N(0,1)^{L_grid x d}``, ``V ~ N(0,1)^{L x d}``, text ``Q, K ~ N(0,1)^{n_text x d}``, and the
  calibration pair indices. Grid rows are ``Q = phi W_Q + 0.3 eps_Q``, ``K = phi W_K + 0.3 eps_K``.
* Optional calibration (FLUX-like layer): grid-token Q and K of a head are multiplied by a
  common ``c > 0`` so that the standard deviation of ``q.k / sqrt(d)`` over 2^16 random grid-token
  pairs equals the target (1.5).
* Values are then rounded to the working dtype (bf16 round-to-nearest-even via torch, or fp32);
  ``to_float64`` gives the exact upcast the oracle consumes.

Each head is generated from its own child stream, so a subset of heads can be produced without
generating the others.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "workload", "custom", "head_inputs", "layer_inputs", "to_float64"]


@dataclasses.dataclass(frozen=True)
class Workload:
    cfg_id: int
    name: str
    H: int
    grid: Tuple[int, ...]
    n_text: int
    d: int
    B: int
    keep: float
    dtype: str  # "f32" or "bf16"
    n_freq: int
    calib_std: Optional[float] = None
    noise: float = 0.3
    freq_scale: float = 2.0 * math.pi
    seed_base: int = 1000

    @property
    def n_grid(self) -> int:
        return int(np.prod(self.grid))

    @property
    def L(self) -> int:
        return self.n_grid + self.n_text

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def describe(self) -> dict:
        return {
            "workload": self.name,
            "H": self.H,
            "L": self.L,
            "grid": list(self.grid),
            "n_text": self.n_text,
            "d": self.d,
            "B": self.B,
            "keep": self.keep,
            "dtype": self.dtype,
        }


# The five synthetic attention layers: tiny CPU-checkable, FLUX-like image, Wan2.1-14B-like 480p
# and 720p video, Hunyuan-Video-like 720p video with text.
WORKLOADS: Sequence[Workload] = (
    Workload(0, "tiny-2d-L1024", H=2, grid=(32, 32), n_text=0, d=64, B=64, keep=0.25,
             dtype="f32", n_freq=16),
    Workload(1, "flux-like-L4608", H=24, grid=(64, 64), n_text=512, d=128, B=64, keep=0.25,
             dtype="bf16", n_freq=16, calib_std=1.5),
    Workload(2, "wan480p-like-L32760", H=40, grid=(21, 30, 52), n_text=0, d=128, B=128,
             keep=0.125, dtype="bf16", n_freq=32),
    Workload(3, "wan720p-like-L75600", H=40, grid=(21, 45, 80), n_text=0, d=128, B=128,
             keep=0.10, dtype="bf16", n_freq=32),
    Workload(4, "hunyuan720p-like-L119056", H=24, grid=(33, 45, 80), n_text=256, d=128, B=128,
             keep=0.08, dtype="bf16", n_freq=32),
)



def workload(name: str) -> Workload:
    """The synthetic layer of that name (see WORKLOADS)."""
    for w in WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(f"unknown workload {name!r}; known: {', '.join(w.name for w in WORKLOADS)}")

def custom(name: str, H: int, grid: Sequence[int], d: int, B: int, keep: float, dtype: str,
           n_text: int = 0, n_freq: Optional[int] = None, calib_std: Optional[float] = None,
           seed: int = 7) -> Workload:
    """A workload with the same recipe at other sizes (tests: ragged tails, tiny shapes)."""
    grid = tuple(int(g) for g in grid)
    if n_freq is None:
        n_freq = 16 if len(grid) <= 2 else 32
    return Workload(cfg_id=seed, name=name, H=H, grid=grid, n_text=n_text, d=d, B=B, keep=keep,
                    dtype=dtype, n_freq=n_freq, calib_std=calib_std)


def _coords(grid: Tuple[int, ...]) -> np.ndarray:
    axes = [np.arange(n, dtype=np.float64) / max(n - 1, 1) for n in grid]
    mesh = np.meshgrid(*axes, indexing="ij")
    return np.stack([m.reshape(-1) for m in mesh], axis=1)  # [n_grid, ndim], raster order


def _children(w: Workload):
    return np.random.SeedSequence(w.seed_base + w.cfg_id).spawn(2 + w.H)


def _features(w: Workload, child) -> np.ndarray:
    rng = np.random.default_rng(child)
    ndim = len(w.grid)
    omega = rng.normal(0.0, w.freq_scale, size=(w.n_freq, ndim))
    b = rng.uniform(0.0, 2.0 * math.pi, size=(w.n_freq,))
    x = _coords(w.grid)
    return math.sqrt(2.0 / w.n_freq) * np.cos(x @ omega.T + b)  # [n_grid, D]


def _round(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(torch.float32 if dtype == "f32" else torch.bfloat16)


def _head_fp64(w: Workload, h: int, phi: np.ndarray, child) -> Tuple[np.ndarray, ...]:
    rng = np.random.default_rng(child)
    D, d, ng, nt = w.n_freq, w.d, w.n_grid, w.n_text
    wq = rng.standard_normal((D, d))
    wk = rng.standard_normal((D, d))
    eq = rng.standard_normal((ng, d))
    ek = rng.standard_normal((ng, d))
    v = rng.standard_normal((w.L, d))
    tq = rng.standard_normal((nt, d))
    tk = rng.standard_normal((nt, d))
    qg = phi @ wq + w.noise * eq
    kg = phi @ wk + w.noise * ek
    if w.calib_std is not None:
        a = rng.integers(0, ng, size=1 << 16)
        c = rng.integers(0, ng, size=1 << 16)
        s = np.einsum("nd,nd->n", qg[a], kg[c]) / math.sqrt(d)
        scale = math.sqrt(w.calib_std / float(np.std(s)))
        qg = qg * scale
        kg = kg * scale
    q = np.concatenate([qg, tq], axis=0)
    k = np.concatenate([kg, tk], axis=0)
    return q, k, v


def head_inputs(w: Workload, h: int, phi: Optional[np.ndarray] = None
                ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Q, K, V of head ``h`` as CPU tensors ``[L, d]`` in the workload dtype."""
    kids = _children(w)
    if phi is None:
        phi = _features(w, kids[0])
    q, k, v = _head_fp64(w, h, phi, kids[2 + h])
    return _round(q, w.dtype), _round(k, w.dtype), _round(v, w.dtype)


def layer_inputs(w: Workload, heads: Optional[Iterable[int]] = None, workers: int = 8):
    """Q, K, V as CPU tensors ``[H', L, d]`` (``H'`` = number of requested heads, default all).
    Heads are generated in a thread pool; each head's values depend only on its own stream."""
    import concurrent.futures as cf

    heads = list(range(w.H)) if heads is None else list(heads)
    L, d = w.L, w.d
    out = [torch.empty((len(heads), L, d), dtype=w.torch_dtype) for _ in range(3)]
    phi = _features(w, _children(w)[0])

    def fill(n_h):
        n, h = n_h
        for dst, src in zip(out, head_inputs(w, h, phi)):
            dst[n].copy_(src)

    with cf.ThreadPoolExecutor(max_workers=max(1, workers)) as ex:
        list(ex.map(fill, enumerate(heads)))
    return tuple(out)


def to_float64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 upcast of a (bf16 or fp32) tensor, as the oracle consumes it."""
    return t.detach().to("cpu").to(torch.float64).numpy()
