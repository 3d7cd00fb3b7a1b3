"""GPU parity of libpisa against the fp64 oracle (through the C ABI).

Bars: selection set-equal per query block except near-ties (oracle score within 1e-5 of the k-th
score); outputs (computed by the oracle with the GPU's own selection) within max-abs 1e-5 for
fp32 inputs, and max-abs 2e-2 plus relative L2 5e-3 for bf16 inputs; statistics to fp32 accuracy.
"""

import numpy as np
import pytest
import torch

from pisa_cases import (assert_close, check_every_head, check_stats, compare_rows, gpu_run, log,
                        oracle_head, sample_blocks)
from workloads import custom, layer_inputs, workload

pytestmark = pytest.mark.gpu


def _full_check(res, heads=None, label="", query_blocks=None, stats=True):
    H = res["out"].shape[0]
    pairs = []
    for h in (range(H) if heads is None else heads):
        ref, out_ref, nsel = oracle_head(res, h, query_blocks=query_blocks)
        if stats and "stats" in res:
            check_stats(res, h, ref)
        qb = range(len(ref["S"])) if query_blocks is None else query_blocks
        pairs.append(compare_rows(res, h, out_ref, qb, res["B"]))
        if nsel:
            log(f"[parity] {label} head {h}: {nsel} rows differ by near-ties only")
    return assert_close(pairs, res["dtype"], label)


# ---------------------------------------------------------------------------------------------
# The tiny fp32 layer, whole: statistics, selection, every output row at 1e-5.
# ---------------------------------------------------------------------------------------------

def test_tiny_fp32_layer():
    w = workload("tiny-2d-L1024")
    res = gpu_run(w, want_stats=True)
    _full_check(res, label=w.name)


@pytest.mark.parametrize("routing", [0, 1])
@pytest.mark.parametrize("phases", [7, 3, 1])
def test_tiny_fp32_modes(routing, phases):
    w = workload("tiny-2d-L1024")
    res = gpu_run(w, routing=routing, phases=phases, want_stats=True)
    _full_check(res, label=f"{w.name} routing={routing} phases={phases}")


# ---------------------------------------------------------------------------------------------
# Small bf16 and fp32 layers covering ragged tails, several tiles, k = 1, k = N_b, L < B.
# ---------------------------------------------------------------------------------------------

SMALL = [
    # name, H, grid, n_text, d, B, keep, dtype
    ("bf16-ragged-3d", 2, (7, 11, 13), 0, 128, 128, 0.3, "bf16"),
    ("bf16-exact-multiple", 2, (16, 16), 0, 128, 128, 0.5, "bf16"),
    ("bf16-B64-text", 3, (20, 30), 100, 128, 64, 0.25, "bf16"),
    ("bf16-k1", 1, (20, 20, 10), 0, 128, 64, 0.01, "bf16"),
    ("bf16-B64-short-tail", 2, (13, 10), 0, 128, 64, 0.5, "bf16"),
    ("bf16-dense", 2, (9, 10, 11), 0, 128, 128, 1.0, "bf16"),
    ("bf16-L-lt-B", 2, (5, 7), 0, 128, 128, 0.5, "bf16"),
    ("bf16-two-pooled-tiles", 2, (9, 30, 65), 0, 128, 128, 0.1, "bf16"),
    ("f32-d128-B128", 2, (7, 11, 13), 0, 128, 128, 0.3, "f32"),
    ("f32-d64-B128", 2, (7, 11, 13), 0, 64, 128, 0.3, "f32"),
    ("f32-d128-B64", 2, (20, 30), 100, 128, 64, 0.25, "f32"),
    ("f32-L-lt-B", 1, (3, 7), 0, 64, 64, 0.5, "f32"),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_layers(case):
    name, H, grid, n_text, d, B, keep, dtype = case
    w = custom(name, H, grid, d, B, keep, dtype, n_text=n_text)
    res = gpu_run(w, want_stats=True)
    _full_check(res, label=name)


@pytest.mark.parametrize("B", [128, 64])
@pytest.mark.parametrize("phases", [3, 1])
@pytest.mark.parametrize("routing", [0, 1])
def test_small_bf16_modes(phases, routing, B):
    w = custom("bf16-modes", 2, (7, 11, 13), 128, B, 0.3, "bf16")
    res = gpu_run(w, routing=routing, phases=phases)
    _full_check(res, label=f"bf16 modes B={B} routing={routing} phases={phases}")


@pytest.mark.parametrize("scale", [0.05, 0.2])
@pytest.mark.parametrize("case", [("bf16", 128, 128), ("bf16", 128, 64), ("f32", 64, 128)],
                         ids=["bf16-B128", "bf16-B64", "f32-d64"])
def test_small_custom_scale(case, scale):
    # a softmax scale other than 1/sqrt(d) (PISA_OPT_SCALE): it enters the Q pre-scale, the pooled
    # queries and scores, and the first-order term
    dtype, d, B = case
    w = custom(f"{dtype}-scale", 2, (7, 11, 13), d, B, 0.3, dtype)
    res = gpu_run(w, scale=scale, want_stats=True)
    _full_check(res, label=f"{dtype} d={d} B={B} scale={scale}")


# ---------------------------------------------------------------------------------------------
# Block-wise first-order variant (per-block H_j instead of H-bar), against the oracle's
# first_order="block" mode; with the first-order phase off the option changes nothing.
# ---------------------------------------------------------------------------------------------

BLOCK_FO = [c for c in SMALL if c[0] in ("bf16-ragged-3d", "bf16-B64-text", "bf16-k1", "bf16-two-pooled-tiles")]


@pytest.mark.parametrize("case", BLOCK_FO, ids=[c[0] for c in BLOCK_FO])
def test_small_block_first_order(case):
    name, H, grid, n_text, d, B, keep, dtype = case
    w = custom(name, H, grid, d, B, keep, dtype, n_text=n_text)
    res = gpu_run(w, want_stats=True, first_order=1)
    _full_check(res, label=f"{name} block first order")


def test_block_first_order_inactive_without_first_phase():
    w = custom("bf16-modes", 2, (7, 11, 13), 128, 128, 0.3, "bf16")
    inputs = layer_inputs(w)
    a = gpu_run(w, inputs=inputs, phases=3)
    b = gpu_run(w, inputs=inputs, phases=3, first_order=1)
    assert torch.equal(a["out"], b["out"])


def test_block_first_order_wan720p():
    w = workload("wan720p-like-L75600")
    res = gpu_run(w, heads=[0, 17], first_order=1)
    qb = sample_blocks(res["info"]["n_blocks"], 6, seed=31)
    _full_check(res, label=f"{w.name} block first order", query_blocks=qb, stats=False)


# ---------------------------------------------------------------------------------------------
# Spectral-norm M_j (covariance routing with the largest singular value of H_j - H-bar).
# ---------------------------------------------------------------------------------------------

def test_tiny_fp32_spectral():
    w = workload("tiny-2d-L1024")
    res = gpu_run(w, want_stats=True, norm=1)
    _full_check(res, label=f"{w.name} spectral")


@pytest.mark.parametrize("case", [c for c in SMALL if c[0] in ("bf16-ragged-3d", "bf16-B64-text", "f32-d64-B128")],
                         ids=["bf16-ragged-3d", "bf16-B64-text", "f32-d64-B128"])
def test_small_spectral(case):
    name, H, grid, n_text, d, B, keep, dtype = case
    w = custom(name, H, grid, d, B, keep, dtype, n_text=n_text)
    res = gpu_run(w, want_stats=True, norm=1)
    _full_check(res, label=f"{name} spectral")


def test_spectral_wan720p_selection():
    w = workload("wan720p-like-L75600")
    res = gpu_run(w, heads=[0, 29], want_stats=True, norm=1)
    qb = sample_blocks(res["info"]["n_blocks"], 6, seed=7)
    _full_check(res, label=f"{w.name} spectral", query_blocks=qb)


# ---------------------------------------------------------------------------------------------
# FLUX-like layer (24 heads, L = 4608, B = 64): every head's selection, four heads' outputs.
# ---------------------------------------------------------------------------------------------

def test_flux_like_layer():
    w = workload("flux-like-L4608")
    res = gpu_run(w, want_stats=True)
    check_every_head(res, label=w.name)
    _full_check(res, heads=[0, 7, 15, 23], label=w.name, stats=False)


# ---------------------------------------------------------------------------------------------
# Full-size video layers, in the launch configuration the benchmark times: every head's complete
# statistics and selection; outputs on sampled query blocks (first, last/ragged, random) of three
# heads, and at Wan-720p every query block of the first and last head.
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["wan480p-like-L32760", "wan720p-like-L75600", "hunyuan720p-like-L119056"])
def test_full_size_layers(name):
    w = workload(name)
    res = gpu_run(w, want_stats=True)
    nb = res["info"]["n_blocks"]
    check_every_head(res, label=w.name)
    heads = [0, w.H // 2, w.H - 1]
    qb = sample_blocks(nb, 10, seed=w.cfg_id)
    _full_check(res, heads=heads, label=w.name, query_blocks=qb, stats=False)
    if name == "wan720p-like-L75600":
        _full_check(res, heads=[0, w.H - 1], label=f"{w.name} every query block of heads 0, {w.H - 1}",
                    stats=False)


# ---------------------------------------------------------------------------------------------
# Large block counts: the routing kernel's N_b > 1024 variants, and the largest supported layer
# (N_b = 8192) with k > 4096, where the attention kernel reads the selection list from global
# memory instead of LDS. Whole selection and statistics of the head; outputs on sampled blocks.
# ---------------------------------------------------------------------------------------------

LARGE = [
    # name, grid, keep
    ("bf16-nb1486-ragged", (29, 83, 79), 0.1),
    ("bf16-nb8192-k4916", (64, 128, 128), 0.6),
]


@pytest.mark.parametrize("case", LARGE, ids=[c[0] for c in LARGE])
def test_large_block_counts(case):
    name, grid, keep = case
    w = custom(name, 1, grid, 128, 128, keep, "bf16")
    res = gpu_run(w, want_stats=True)
    nb = res["info"]["n_blocks"]
    log(f"[parity] {name}: N_b={nb} k={res['info']['k']}")
    _full_check(res, heads=[0], label=name, query_blocks=sample_blocks(nb, 4, seed=nb))


# ---------------------------------------------------------------------------------------------
# Determinism and stage equivalence.
# ---------------------------------------------------------------------------------------------

def test_deterministic_and_stages_match_forward():
    w = workload("flux-like-L4608")
    inputs = layer_inputs(w, heads=range(6))
    a = gpu_run(w, inputs=inputs)
    b = gpu_run(w, inputs=inputs)
    c = gpu_run(w, inputs=inputs, stages=True)
    assert torch.equal(a["out"], b["out"]) and np.array_equal(a["idx"], b["idx"])
    assert torch.equal(a["out"], c["out"]) and np.array_equal(a["idx"], c["idx"])


def test_two_plans_on_side_streams():
    # two plans (own workspaces) run concurrently on two non-default streams; each gives the same
    # bits as a plan on the current stream
    from sparse_attention_diffusion_pool_amd import _lib as L
    w = custom("bf16-streams", 2, (7, 11, 13), 128, 128, 0.3, "bf16")
    dev = torch.device("cuda", 0)
    qd, kd, vd = (t.to(dev) for t in layer_inputs(w))
    H, Lq, d = qd.shape
    plans = [L.Plan(Lq, H, d, w.B, w.keep, dtype=L.DTYPE_BF16) for _ in range(3)]
    for p in plans:
        p.attach_workspace(device=dev)
    outs = [torch.full_like(qd, float("nan")) for _ in range(3)]
    plans[0].forward(qd, kd, vd, outs[0])
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for s, p, o in zip(streams, plans[1:], outs[1:]):
        with torch.cuda.stream(s):
            p.forward(qd, kd, vd, o, stream=s)
    torch.cuda.synchronize()
    for p in plans:
        p.destroy()
    assert torch.isfinite(outs[0].float()).all()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


def test_graph_capture_replays():
    # pisa_forward launches kernels only (no allocation, no memset), so it can be captured in a
    # HIP graph. Each replay follows eager work that changes Q in place, and must match an eager
    # forward of a second plan on the same inputs bit for bit.
    from sparse_attention_diffusion_pool_amd import _lib as L
    w = custom("bf16-graph", 2, (7, 11, 13), 128, 128, 0.3, "bf16")
    dev = torch.device("cuda", 0)
    qd, kd, vd = (t.to(dev) for t in layer_inputs(w))
    H, Lq, d = qd.shape
    plan_g, plan_e = (L.Plan(Lq, H, d, w.B, w.keep, dtype=L.DTYPE_BF16) for _ in range(2))
    plan_g.attach_workspace(device=dev)
    plan_e.attach_workspace(device=dev)
    out_g, ref = torch.empty_like(qd), torch.empty_like(qd)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan_g.forward(qd, kd, vd, out_g)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan_g.forward(qd, kd, vd, out_g)
    torch.cuda.synchronize()
    for r in range(4):
        qd.mul_(1.0 + 0.25 * r)  # eager work between replays
        plan_e.forward(qd, kd, vd, ref)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(ref.float()).all()
        assert torch.equal(out_g, ref), f"replay {r} differs from the eager forward"
    del graph
    plan_g.destroy()
    plan_e.destroy()


def test_outputs_untouched_outside_rows_and_no_nan():
    # out is pre-filled with NaN by gpu_run: every row must be written, none left NaN
    w = custom("fill", 2, (7, 11, 13), 128, 128, 0.3, "bf16")
    res = gpu_run(w)
    assert torch.isfinite(res["out"].float()).all()


# ---------------------------------------------------------------------------------------------
# Measurement support: the MFMA probe runs, its results are finite and its clock reading sane.
# ---------------------------------------------------------------------------------------------

def test_mfma_probe():
    from sparse_attention_diffusion_pool_amd import _lib as L
    blocks, iters = 256, 200
    dev = torch.device("cuda", 0)
    out = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device=dev)
    clk = torch.zeros(blocks * 2, dtype=torch.int64, device=dev)
    L.mfma_probe(out, clk, blocks, iters)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.isfinite(o).all() and (o > 0).all()
    c = clk.view(blocks, 2).cpu().numpy().astype(np.float64)
    assert (c > 0).all()
    ghz = c[:, 0].sum() / c[:, 1].sum() * 0.1  # shader ticks per 100 MHz tick
    log(f"[probe] shader clock {ghz:.3f} GHz over {blocks} workgroups")
    assert 0.5 < ghz < 3.0
