"""Shared helpers of the GPU parity tests: run libpisa on a seeded workload, then compare with the
fp64 oracle (statistics, selection, outputs)."""

from __future__ import annotations

import math
import sys

import numpy as np
import torch

from oracle import pisa_oracle as po
from sparse_attention_diffusion_pool_amd import _lib as L
from workloads import layer_inputs, to_float64

# Output bars: fp32 inputs max-abs 1e-5; bf16 inputs max-abs 2e-2 and relative L2 5e-3.
TOL = {"f32": {"max_abs": 1e-5, "rel_l2": None}, "bf16": {"max_abs": 2e-2, "rel_l2": 5e-3}}
# Selection: GPU and oracle sets must agree except for blocks whose oracle score lies within this
# distance of the oracle's k-th score (the GPU ranks fp32 scores).
NEAR_TIE = 1e-5

PHASES = {7: {"first_order": "global", "drop": False},
          3: {"first_order": "none", "drop": False},
          1: {"first_order": "global", "drop": True}}


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def gpu_run(w, heads=None, keep=None, B=None, routing=0, phases=7, inputs=None, want_stats=False,
            stages=False, first_order=0, norm=0, scale=None):
    q, k, v = inputs if inputs is not None else layer_inputs(w, heads)
    H, Lq, d = q.shape
    B = w.B if B is None else B
    keep = w.keep if keep is None else keep
    dev = torch.device("cuda", 0)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    dtype = L.DTYPE_BF16 if q.dtype == torch.bfloat16 else L.DTYPE_F32
    plan = L.Plan(Lq, H, d, B, keep, dtype=dtype, routing=routing, phases=phases, first_order=first_order,
                  norm=norm, scale=scale)
    plan.attach_workspace(device=dev)
    info = plan.info()
    out = torch.full_like(qd, float("nan"))
    log(f"[gpu] {w.name} H={H} L={Lq} d={d} B={B} keep={keep} k={info['k']} routing={routing} "
        f"phases={phases} stages={stages} first_order={first_order} norm={norm} scale={scale}")
    if stages:
        plan.forward_stats(qd, kd, vd)
        plan.forward_route()
        plan.forward_attend(qd, kd, vd, out)
    else:
        plan.forward(qd, kd, vd, out)
    nb, kk = info["n_blocks"], info["k"]
    idx = torch.empty((H, nb, kk), dtype=torch.int32, device=dev)
    plan.debug_copy_selection(idx)
    stats = None
    if want_stats:
        f = dict(dtype=torch.float32, device=dev)
        stats = {"qbar": torch.empty((H, nb, d), **f), "kbar": torch.empty((H, nb, d), **f),
                 "vsum": torch.empty((H, nb, d), **f), "hbar": torch.empty((H, d, d), **f),
                 "M": torch.empty((H, nb), **f)}
        plan.debug_copy_stats(**stats)
    torch.cuda.synchronize()
    log(f"[gpu] done {w.name}")
    res = {"out": out.cpu(), "idx": idx.cpu().numpy(), "info": info, "inputs": (q, k, v), "B": B,
           "keep": keep, "routing": routing, "phases": phases, "dtype": w.dtype, "first_order": first_order,
           "norm": norm, "scale": scale}
    if stats is not None:
        res["stats"] = {n: t.cpu().numpy().astype(np.float64) for n, t in stats.items()}
    plan.destroy()
    return res


def check_selection(gidx: np.ndarray, scores: np.ndarray, S_ref, kk: int) -> int:
    """GPU selection of one head vs the oracle's; returns the number of rows that differ (all by
    near-ties only, else AssertionError)."""
    nb = scores.shape[0]
    differ = 0
    for i in range(nb):
        g = gidx[i]
        assert np.all(np.diff(g) > 0), f"row {i}: indices not strictly ascending: {g}"
        assert g[0] >= 0 and g[-1] < nb
        gs, os_ = set(int(x) for x in g), set(int(x) for x in S_ref[i])
        if gs == os_:
            continue
        differ += 1
        kth = np.sort(scores[i])[::-1][kk - 1]
        for j in gs ^ os_:
            assert abs(scores[i][j] - kth) < NEAR_TIE, (
                f"row {i}: block {j} differs, score {scores[i][j]!r} vs k-th {kth!r}")
    return differ


def oracle_head(res, h: int, query_blocks=None):
    """Oracle statistics/selection for head h, and the oracle output on query_blocks computed with
    the GPU's own selection."""
    q, k, v = (to_float64(t[h]) for t in res["inputs"])
    B, keep = res["B"], res["keep"]
    routing = "cov" if res["routing"] == 0 else "plain"
    mode = dict(PHASES[res["phases"]])
    if res.get("first_order") == 1 and res["phases"] == 7:
        mode["first_order"] = "block"
    mode["norm"] = "spectral" if res.get("norm") == 1 else "fro"
    scale = res.get("scale")
    ref = po.pisa_head(q, k, v, B, keep, scale=scale, routing=routing, query_blocks=[], **mode)
    nsel = check_selection(res["idx"][h], ref["scores"], ref["S"], ref["k"])
    qb = range(len(ref["S"])) if query_blocks is None else query_blocks
    gsel = [list(map(int, s)) for s in res["idx"][h]]
    out_ref = po.pisa_head(q, k, v, B, keep, scale=scale, routing=routing, selection=gsel, query_blocks=qb,
                           **mode)["out"]
    return ref, out_ref, nsel


def compare_rows(res, h: int, out_ref: np.ndarray, query_blocks, B: int):
    L_ = out_ref.shape[0]
    rows = np.concatenate([np.arange(i * B, min(L_, (i + 1) * B)) for i in query_blocks])
    g = res["out"][h].to(torch.float64).numpy()[rows]
    r = out_ref[rows]
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    return g, r


def assert_close(pairs, dtype: str, label: str):
    g = np.concatenate([p[0].ravel() for p in pairs])
    r = np.concatenate([p[1].ravel() for p in pairs])
    max_abs = float(np.max(np.abs(g - r)))
    rel_l2 = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))
    tol = TOL[dtype]
    log(f"[parity] {label}: max_abs={max_abs:.3e} rel_l2={rel_l2:.3e} (bar {tol})")
    assert max_abs <= tol["max_abs"], f"{label}: max_abs {max_abs} > {tol['max_abs']}"
    if tol["rel_l2"] is not None:
        assert rel_l2 <= tol["rel_l2"], f"{label}: rel_l2 {rel_l2} > {tol['rel_l2']}"
    return max_abs, rel_l2


def check_stats(res, h: int, ref):
    st = ref["stats"]
    gs = {n: a[h] for n, a in res["stats"].items()}
    for name, gv, rv in (("qbar", gs["qbar"], st.qbar), ("kbar", gs["kbar"], st.kbar), ("vsum", gs["vsum"], st.vsum)):
        scale = np.max(np.abs(rv)) + 1e-30
        err = np.max(np.abs(gv - rv)) / scale
        assert err < 2e-6, f"{name}: rel err {err}"
    hscale = np.max(np.abs(st.H))
    err_h = np.max(np.abs(gs["hbar"] - st.Hbar)) / hscale
    assert err_h < 2e-6, f"hbar: err/max|H_j| {err_h}"
    if res["routing"] == 0:
        # relative where M_j is large; where it vanishes (one block: H_0 = H-bar) the GPU value is
        # fp32 rounding of a difference of matrices of norm ~||H_j||_F, so the floor scales with it
        hnorm = np.max(np.sqrt(np.einsum("jab,jab->j", st.H, st.H)))
        err_m = np.max(np.abs(gs["M"] - st.M) / (st.M + 0.05 * hnorm))
        assert err_m < 2e-5, f"M: rel err {err_m}"


def check_every_head(res, heads=None, workers: int = 8, label: str = ""):
    """Statistics (if copied) and selection of every head against the oracle, in a thread pool
    (NumPy releases the GIL in its kernels). Logs and returns the near-tie row count per head."""
    import concurrent.futures as cf

    heads = list(range(res["out"].shape[0])) if heads is None else list(heads)

    def one(h):
        ref, _, nsel = oracle_head(res, h, query_blocks=[])
        if "stats" in res:
            check_stats(res, h, ref)
        return h, nsel

    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        ties = dict(ex.map(one, heads))
    log(f"[parity] {label}: statistics and selection of {len(heads)} heads match; near-tie rows per "
        f"head: {[ties[h] for h in heads]}")
    return ties


def sample_blocks(nb: int, n: int, seed: int):
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(nb, size=min(n, nb), replace=False).tolist())
    pick |= {0, nb - 1}
    return sorted(pick)
