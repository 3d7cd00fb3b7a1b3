"""Pins of the fp64 oracle against what the pages and the mathematics fix (no GPU).

Each test states what it pins. None of them re-types the oracle's formulas in the same form:
dense attention comes from torch's SDPA in float64, the Taylor expansion from element loops in
oracle/brute.py, H-bar from a whole-matrix identity, top-k from torch.topk.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import brute
from oracle import pisa_oracle as po
from workloads import custom, head_inputs, to_float64, workload


def _sdpa(q, k, v, scale, mask=None):
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x))[None, None] for x in (q, k, v))
    am = None if mask is None else torch.from_numpy(mask)[None, None]
    return F.scaled_dot_product_attention(tq, tk, tv, attn_mask=am, scale=scale)[0, 0].numpy()


def _rand(L, d, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return [scale * rng.standard_normal((L, d)) for _ in range(3)]


def _lists(*xs):
    return [x.tolist() for x in xs]


# --- P1: keep = 1 selects every block, U is empty, the output is dense softmax attention ---------

@pytest.mark.parametrize("L,d,B", [(200, 16, 64), (1024, 64, 64), (131, 8, 16)])
def test_keep_all_equals_dense(L, d, B):
    q, k, v = _rand(L, d, seed=L + d)
    r = po.pisa_head(q, k, v, B, keep=1.0)
    assert all(len(s) == po.n_blocks(L, B) for s in r["S"])
    ref = _sdpa(q, k, v, 1.0 / math.sqrt(d))
    assert np.max(np.abs(r["out"] - ref)) < 1e-10


def test_keep_all_equals_dense_tiny_config():
    w = workload("tiny-2d-L1024")
    q, k, v = (to_float64(t) for t in head_inputs(w, 0))
    r = po.pisa_head(q, k, v, w.B, keep=1.0)
    ref = _sdpa(q, k, v, 1.0 / math.sqrt(w.d))
    assert np.max(np.abs(r["out"] - ref)) < 1e-10


# --- P2: B = 1 -> every block is one token: kbar_j = k_j, H_j = 0, the expansion is exact ----------

@pytest.mark.parametrize("keep", [0.05, 0.3, 0.7])
def test_block_size_one_is_dense(keep):
    q, k, v = _rand(48, 8, seed=3)
    r = po.pisa_head(q, k, v, 1, keep=keep)
    assert np.max(np.abs(r["stats"].H)) < 1e-14
    ref = _sdpa(q, k, v, 1.0 / math.sqrt(8))
    assert np.max(np.abs(r["out"] - ref)) < 1e-12


# --- P3: keys constant inside every block -> q~.k constant per block, H_j = 0 -> dense -------------

@pytest.mark.parametrize("routing", ["cov", "plain"])
@pytest.mark.parametrize("keep", [0.1, 0.5])
def test_constant_key_blocks_are_dense(routing, keep):
    L, d, B = 150, 16, 16
    rng = np.random.default_rng(11)
    q = rng.standard_normal((L, d))
    v = rng.standard_normal((L, d))
    kb = rng.standard_normal((po.n_blocks(L, B), d))
    k = np.repeat(kb, B, axis=0)[:L]
    r = po.pisa_head(q, k, v, B, keep=keep, routing=routing)
    assert np.max(np.abs(r["stats"].H)) < 1e-12
    ref = _sdpa(q, k, v, 1.0 / math.sqrt(d))
    assert np.max(np.abs(r["out"] - ref)) < 1e-12


def test_cov_routing_reduces_to_plain_when_blocks_are_homogeneous():
    # every M_j = 0 and every n_j equal: ln(n_j + |qbar| M_j) is a per-row constant
    L, d, B = 160, 8, 16
    rng = np.random.default_rng(5)
    q = rng.standard_normal((L, d))
    v = rng.standard_normal((L, d))
    k = np.repeat(rng.standard_normal((L // B, d)), B, axis=0)
    st = po.head_stats(q, k, v, B, 1 / math.sqrt(d))
    assert np.max(st.M) < 1e-12
    kk = 3
    a = po.select_blocks(po.routing_scores(st, "cov"), kk)
    b = po.select_blocks(po.routing_scores(st, "plain"), kk)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


# --- covariance-aware routing term (gist.science summary, section 2 "Covariance-aware routing") ----
# The pages name the score's ingredients (the attention score and M_j = ||H_j - H-bar||) without a
# formula; the reading ranks block j by its zeroth-order mass n_j alpha plus the bound
# alpha ||q~|| M_j on the first-order numerator error, in logs at the pooled query. The three pins
# below each isolate one ingredient with quantities computed outside the oracle.

def test_cov_minus_plain_is_log_count_with_flat_blocks():
    # keys constant inside every block: H_j = 0 = H-bar, M_j = 0, so the covariance term is ln n_j,
    # with n_j = B for full blocks and L - (N_b - 1) B for the ragged last one
    L, d, B = 150, 8, 16
    rng = np.random.default_rng(41)
    nb = -(-L // B)
    q = 0.7 + rng.standard_normal((L, d))
    v = rng.standard_normal((L, d))
    k = np.repeat(rng.standard_normal((nb, d)), B, axis=0)[:L]
    st = po.head_stats(q, k, v, B, 1 / math.sqrt(d))
    gap = po.routing_scores(st, "cov") - po.routing_scores(st, "plain")
    counts = np.array([B] * (nb - 1) + [L - (nb - 1) * B], dtype=np.float64)
    assert counts[-1] == 6
    assert np.max(np.abs(gap - np.log(counts)[None, :])) < 1e-12


def _equal_centroid_layer(seed=43):
    # blocks 0 and 1 share their centroid c; block 0's keys spread along its values (large H_0),
    # block 1's keys are all c (H_1 = 0); blocks 2..4 are random, block 4 ragged
    L, d, B = 72, 8, 16
    rng = np.random.default_rng(seed)
    q = 1.0 + rng.standard_normal((L, d))
    v = rng.standard_normal((L, d))
    k = rng.standard_normal((L, d))
    c = rng.standard_normal(d)
    spread = 3.0 * v[0:B, :d]
    spread -= spread.mean(axis=0)
    k[0:B] = c + spread
    k[B:2 * B] = c
    return q, k, v, B, 1 / math.sqrt(d)


def test_cov_score_gap_between_equal_centroids():
    # equal q.kbar: the score gap is the covariance term alone, ln((n + |qbar_i| M_0)/(n + |qbar_i| M_1)),
    # with |qbar_i| the Euclidean norm of the scaled pooled query (taken here from q directly) and
    # M_j from the element loops; the block with the larger M_j ranks higher in every row
    q, k, v, B, tau = _equal_centroid_layer()
    L, d = q.shape
    st = po.head_stats(q, k, v, B, tau)
    sc = po.routing_scores(st, "cov")
    bs = brute.block_stats(*_lists(q, k, v), B, tau)
    M0, M1 = bs["M"][0], bs["M"][1]
    assert M0 > 2 * M1 > 0
    for i, (s0, e0) in enumerate(po.block_bounds(L, B)):
        qn = math.sqrt(sum((tau * sum(q[r][c] for r in range(s0, e0)) / (e0 - s0)) ** 2 for c in range(d)))
        want = math.log((B + qn * M0) / (B + qn * M1))
        assert abs((sc[i, 0] - sc[i, 1]) - want) < 1e-10
        assert sc[i, 0] > sc[i, 1]


@pytest.mark.parametrize("norm", ["fro", "spectral"])
def test_cov_m_bounds_first_order_error(norm):
    # M_j bounds the first-order numerator error of routing j to U at any query:
    # |q (H_j - H-bar)| <= |q| M_j, for the pooled queries and for every token's scaled query
    q, k, v, B, tau = _equal_centroid_layer(seed=47)
    st = po.head_stats(q, k, v, B, tau, norm=norm)
    bs = brute.block_stats(*_lists(q, k, v), B, tau)
    E = np.array(bs["H"]) - np.array(bs["Hbar"])[None]
    for x in list(st.qbar) + list(tau * q):
        lhs = np.linalg.norm(np.einsum("a,jab->jb", x, E), axis=1)
        assert np.all(lhs <= np.linalg.norm(x) * st.M * (1 + 1e-12) + 1e-12)


# --- P4: the centroid is the mean, so the denominator's first-order sum vanishes -----------------

def test_denominator_first_order_vanishes():
    q, k, v = _rand(77, 8, seed=9)
    B = 10
    st = po.head_stats(q, k, v, B, 1 / math.sqrt(8))
    for j, (s, e) in enumerate(po.block_bounds(77, B)):
        dev = (k[s:e] - st.kbar[j]).sum(axis=0)
        assert np.max(np.abs(dev)) <= 1e-12 * np.abs(k[s:e]).sum()
        assert st.n[j] == e - s


# --- P5: brute-force element loops on tiny inputs -----------------------------------------------

CASES = [(12, 4, 4, 0.5), (23, 4, 5, 0.4), (37, 4, 5, 0.25), (48, 3, 4, 0.2)]


@pytest.mark.parametrize("L,d,B,keep", CASES)
def test_block_stats_match_loops(L, d, B, keep):
    q, k, v = _rand(L, d, seed=L)
    tau = 1 / math.sqrt(d)
    st = po.head_stats(q, k, v, B, tau)
    bs = brute.block_stats(*_lists(q, k, v), B, tau)
    assert np.allclose(st.kbar, bs["kbar"], atol=1e-13, rtol=0)
    assert np.allclose(st.vsum, bs["vsum"], atol=1e-13, rtol=0)
    assert np.allclose(st.qbar, bs["qbar"], atol=1e-13, rtol=0)
    assert np.allclose(st.H, bs["H"], atol=1e-12, rtol=0)
    assert np.allclose(st.Hbar, bs["Hbar"], atol=1e-12, rtol=0)
    assert np.allclose(st.M, bs["M"], atol=1e-12, rtol=0)


@pytest.mark.parametrize("routing", ["cov", "plain"])
@pytest.mark.parametrize("L,d,B,keep", CASES)
def test_routing_matches_sort(L, d, B, keep, routing):
    q, k, v = _rand(L, d, seed=2 * L + 1)
    tau = 1 / math.sqrt(d)
    r = po.pisa_head(q, k, v, B, keep, routing=routing)
    bs = brute.block_stats(*_lists(q, k, v), B, tau)
    S, scores = brute.route(bs, r["k"], routing)
    assert np.allclose(r["scores"], scores, atol=1e-12, rtol=0)
    assert [list(x) for x in r["S"]] == S


@pytest.mark.parametrize("first_order", ["global", "block", "none"])
@pytest.mark.parametrize("drop", [False, True])
@pytest.mark.parametrize("L,d,B,keep", CASES)
def test_output_matches_elementwise_taylor(L, d, B, keep, first_order, drop):
    q, k, v = _rand(L, d, seed=L * 7 + d, scale=0.8)
    tau = 1 / math.sqrt(d)
    r = po.pisa_head(q, k, v, B, keep, first_order=first_order, drop=drop)
    S = [list(map(int, s)) for s in r["S"]]
    bt = np.array(brute.taylor_rows(*_lists(q, k, v), B, tau, S, first_order=first_order, drop=drop))
    assert np.max(np.abs(r["out"] - bt)) < 1e-12


def test_global_minus_block_first_order_closed_form():
    # PISA - (same with per-block H_j) = sum_{j in U} alpha_{t,j} q~ (Hbar - H_j) / D_t
    L, d, B, keep = 37, 4, 5, 0.25
    q, k, v = _rand(L, d, seed=123)
    tau = 1 / math.sqrt(d)
    g = po.pisa_head(q, k, v, B, keep, first_order="global")
    b = po.pisa_head(q, k, v, B, keep, first_order="block")
    bs = brute.block_stats(*_lists(q, k, v), B, tau)
    nb = len(bs["n"])
    for i, (s0, e0) in enumerate(bs["blocks"]):
        U = [j for j in range(nb) if j not in set(g["S"][i])]
        for t in range(s0, e0):
            qt = tau * q[t]
            # unshifted denominator from brute quantities
            D = sum(math.exp(qt @ k[r]) for j in g["S"][i] for r in range(*bs["blocks"][j]))
            D += sum(bs["n"][j] * math.exp(qt @ np.array(bs["kbar"][j])) for j in U)
            corr = sum(math.exp(qt @ np.array(bs["kbar"][j]))
                       * (qt @ (np.array(bs["Hbar"]) - np.array(bs["H"][j]))) for j in U)
            assert np.max(np.abs((g["out"][t] - b["out"][t]) - corr / D)) < 1e-12


# --- spectral reading of M_j: power iteration on tiny blocks, rank-1 and norm-ordering checks -------

@pytest.mark.parametrize("L,d,B,keep", CASES)
def test_spectral_m_matches_power_iteration(L, d, B, keep):
    q, k, v = _rand(L, d, seed=5 * L + 3)
    tau = 1 / math.sqrt(d)
    st = po.head_stats(q, k, v, B, tau, norm="spectral")
    fro = po.head_stats(q, k, v, B, tau).M
    bs = brute.block_stats(*_lists(q, k, v), B, tau)
    for j in range(len(st.n)):
        E = [[bs["H"][j][a][b] - bs["Hbar"][a][b] for b in range(d)] for a in range(d)]
        assert abs(st.M[j] - brute.spectral_norm(E)) <= 1e-9 * max(1.0, fro[j])
        assert st.M[j] <= fro[j] * (1 + 1e-12) and fro[j] <= math.sqrt(d) * st.M[j] * (1 + 1e-12)


def test_spectral_equals_frobenius_for_rank_one():
    # one key direction per block and H-bar = 0 make every H_j - H-bar rank one
    L, d, B = 64, 6, 8
    rng = np.random.default_rng(17)
    dirn = rng.standard_normal(d)
    k = np.outer(rng.standard_normal(L), dirn)
    k -= np.repeat(k.reshape(-1, B, d).mean(axis=1), B, axis=0)  # zero-mean blocks: H_j = K_j^T V_j
    v = rng.standard_normal((L, d))
    v[L // 2:] = -v[:L // 2][::-1]  # ... and K_j^T V_j of mirrored halves cancel in H-bar
    k[L // 2:] = k[:L // 2][::-1]
    st_s = po.head_stats(rng.standard_normal((L, d)), k, v, B, 1.0, norm="spectral")
    st_f = po.head_stats(rng.standard_normal((L, d)), k, v, B, 1.0)
    assert np.max(np.abs(st_f.Hbar)) < 1e-12
    assert np.allclose(st_s.M, st_f.M, rtol=1e-12, atol=1e-12)


# --- P6: H-bar identity from whole-matrix products ------------------------------------------------

def test_hbar_identity():
    w = workload("tiny-2d-L1024")
    q, k, v = (to_float64(t) for t in head_inputs(w, 1))
    st = po.head_stats(q, k, v, w.B, 1 / math.sqrt(w.d))
    nb = po.n_blocks(w.L, w.B)
    corr = sum(np.outer(st.kbar[j], st.vsum[j]) for j in range(nb))  # n_j kbar_j vbar_j^T
    ident = (k.T @ v - corr) / nb
    assert np.max(np.abs(st.Hbar - ident)) < 1e-11


# --- P7: no critical blocks, no first order -> softmax over pooled tokens with bias ln n_j --------

def test_pooled_tokens_are_biased_softmax():
    L, d, B = 150, 16, 16
    q, k, v = _rand(L, d, seed=21)
    nb = po.n_blocks(L, B)
    r = po.pisa_head(q, k, v, B, keep=0.5, selection=[[] for _ in range(nb)], first_order="none")
    n = np.array([e - s for s, e in po.block_bounds(L, B)], dtype=np.float64)
    kbar = np.stack([k[s:e].mean(0) for s, e in po.block_bounds(L, B)])
    vbar = np.stack([v[s:e].mean(0) for s, e in po.block_bounds(L, B)])
    mask = np.broadcast_to(np.log(n)[None, :], (L, nb)).copy()
    ref = _sdpa(q, kbar, vbar, 1 / math.sqrt(d), mask)
    assert np.max(np.abs(r["out"] - ref)) < 1e-12


# --- P8: Jensen ordering of the partition function for a fixed selection --------------------------

def test_jensen_ordering():
    w = custom("j", 1, (12, 12), 16, 16, 0.25, "f32")
    q, k, v = (to_float64(t) for t in head_inputs(w, 0))
    tau = 1 / math.sqrt(w.d)
    st = po.head_stats(q, k, v, w.B, tau)
    S = po.select_blocks(po.routing_scores(st), po.top_k_count(w.keep, len(st.n)))
    for i, (s0, e0) in enumerate(po.block_bounds(w.L, w.B)):
        qt = tau * q[s0:e0]
        _, _, Dp, mp = po.piecewise_rows(qt, k, v, st, S[i], w.B, return_parts=True)
        _, _, Dd, md = po.piecewise_rows(qt, k, v, st, S[i], w.B, drop=True, return_parts=True)
        logz_dense = np.log(np.exp(qt @ k.T).sum(axis=1))
        lp, ld = np.log(Dp) + mp, np.log(Dd) + md
        assert np.all(ld <= lp + 1e-12) and np.all(lp <= logz_dense + 1e-12)
        assert np.all(lp < logz_dense)  # strict: keys vary inside every block


# --- P9: translation and linearity invariants ---------------------------------------------------

def test_value_translation_and_linearity():
    L, d, B = 130, 8, 16
    q, k, v = _rand(L, d, seed=31)
    c = np.linspace(-1, 2, d)
    a = po.pisa_head(q, k, v, B, 0.3)
    b = po.pisa_head(q, k, v + c[None, :], B, 0.3)
    assert [list(x) for x in a["S"]] == [list(x) for x in b["S"]]
    assert np.max(np.abs(b["out"] - (a["out"] + c))) < 1e-12
    v2 = np.random.default_rng(1).standard_normal((L, d))
    sel = a["S"]
    o1 = po.pisa_head(q, k, v, B, 0.3, selection=sel)["out"]
    o2 = po.pisa_head(q, k, v2, B, 0.3, selection=sel)["out"]
    o3 = po.pisa_head(q, k, v - 2.5 * v2, B, 0.3, selection=sel)["out"]
    assert np.max(np.abs(o3 - (o1 - 2.5 * o2))) < 1e-12


def test_key_translation():
    L, d, B = 130, 8, 16
    q, k, v = _rand(L, d, seed=33)
    c = np.linspace(1, -1, d)
    a = po.pisa_head(q, k, v, B, 0.3)
    b = po.pisa_head(q, k + c[None, :], v, B, 0.3)
    assert [list(x) for x in a["S"]] == [list(x) for x in b["S"]]
    assert np.max(np.abs(b["out"] - a["out"])) < 1e-12


# --- P10: plain routing is the textbook top-k of the pooled product; ties go to the lower index ---

def test_plain_routing_is_topk():
    w = workload("tiny-2d-L1024")
    q, k, v = (to_float64(t) for t in head_inputs(w, 0))
    tau = 1 / math.sqrt(w.d)
    r = po.pisa_head(q, k, v, w.B, w.keep, routing="plain")
    tq = torch.from_numpy(tau * q).view(-1, w.B, w.d).mean(1)
    tk = torch.from_numpy(k).view(-1, w.B, w.d).mean(1)
    top = torch.topk(tq @ tk.T, r["k"], dim=1).indices.sort(dim=1).values
    assert np.array_equal(np.stack(r["S"]), top.numpy())


def test_ties_go_to_lower_index():
    L, d, B = 96, 4, 8
    q, _, v = _rand(L, d, seed=1)
    k = np.zeros((L, d))
    r = po.pisa_head(q, k, v, B, keep=0.25, routing="plain")
    assert all(list(s) == [0, 1, 2] for s in r["S"])


def test_top_k_count():
    assert po.top_k_count(0.25, 16) == 4
    assert po.top_k_count(0.10, 591) == 60
    assert po.top_k_count(0.08, 931) == 75
    assert po.top_k_count(0.125, 256) == 32
    assert po.top_k_count(0.25, 72) == 18
    assert po.top_k_count(1e-6, 10) == 1
    assert po.top_k_count(1.0, 10) == 10


def test_executed_flops_dense_limit():
    # keep = 1: exact part = 4 L^2 d (QK^T and PV), no zeroth-order part
    L, d, B = 300, 8, 64
    nb = po.n_blocks(L, B)
    f = po.executed_flops(L, d, B, [list(range(nb))] * nb)
    assert f["exact"] == 4 * L * L * d and f["zeroth"] == 0


# --- stored regression anchor written by tests/golden/make_golden.py (oracle code only) -----------

def test_golden_tiny_taylor():
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_taylor.json")
    g = json.load(open(path))
    q, k, v = (np.array(g[x]) for x in ("q", "k", "v"))
    for fo in ("global", "block", "none"):
        r = po.pisa_head(q, k, v, g["B"], g["keep"], first_order=fo)
        assert [list(map(int, s)) for s in r["S"]] == g["S"]
        assert np.max(np.abs(r["out"] - np.array(g["out"][fo]))) < 1e-12
    r = po.pisa_head(q, k, v, g["B"], g["keep"], drop=True)
    assert np.max(np.abs(r["out"] - np.array(g["out"]["drop"]))) < 1e-12
