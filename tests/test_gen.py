"""Seeded generator: reproducibility, shapes, token order, calibration (no method arithmetic)."""

import math

import numpy as np
import torch

from workloads import WORKLOADS, custom, head_inputs, layer_inputs, to_float64, workload


def test_config_shapes():
    want = {0: (2, 1024, 64, 64, "f32"), 1: (24, 4608, 128, 64, "bf16"),
            2: (40, 32760, 128, 128, "bf16"), 3: (40, 75600, 128, 128, "bf16"),
            4: (24, 119056, 128, 128, "bf16")}
    for w in WORKLOADS:
        assert (w.H, w.L, w.d, w.B, w.dtype) == want[w.cfg_id]


def test_reproducible_and_head_independent():
    w = workload("tiny-2d-L1024")
    a = head_inputs(w, 1)
    b = head_inputs(custom("other", 1, (4, 4), 8, 4, 0.5, "f32"), 0)  # evict the cache
    c = head_inputs(w, 1)
    for x, y in zip(a, c):
        assert torch.equal(x, y)
    q, k, v = layer_inputs(w)
    assert torch.equal(q[1], a[0]) and torch.equal(k[1], a[1]) and torch.equal(v[1], a[2])
    assert not torch.equal(q[0], q[1])
    assert b[0].shape == (16, 8)


def test_dtypes_and_rounding():
    w = custom("bf", 1, (8, 8), 128, 64, 0.25, "bf16")
    q, k, v = head_inputs(w, 0)
    assert q.dtype == torch.bfloat16
    q64 = to_float64(q)
    # exact upcast: rounding back gives the same bits
    assert torch.equal(torch.from_numpy(q64).to(torch.bfloat16), q)


def test_text_tokens_at_tail_iid():
    w = custom("txt", 2, (16, 16), 128, 64, 0.25, "bf16", n_text=512, n_freq=16)
    q, k, v = head_inputs(w, 0)
    t = to_float64(q[256:])
    assert abs(t.mean()) < 0.02 and abs(t.std() - 1.0) < 0.02
    # grid tokens are spatially smooth: neighbouring rows correlate, text rows do not
    g = to_float64(k[:256])
    nb = np.corrcoef(g[:-1].ravel(), g[1:].ravel())[0, 1]
    tt = to_float64(k[256:])
    nt = np.corrcoef(tt[:-1].ravel(), tt[1:].ravel())[0, 1]
    assert nb > 0.5 and abs(nt) < 0.05


def test_flux_calibration_std():
    w = workload("flux-like-L4608")
    q, k, _ = head_inputs(w, 3)
    qg, kg = to_float64(q[: w.n_grid]), to_float64(k[: w.n_grid])
    rng = np.random.default_rng(0)
    a = rng.integers(0, w.n_grid, 1 << 16)
    b = rng.integers(0, w.n_grid, 1 << 16)
    s = np.einsum("nd,nd->n", qg[a], kg[b]) / math.sqrt(w.d)
    assert abs(s.std() - 1.5) / 1.5 < 0.02
