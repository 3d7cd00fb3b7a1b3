"""fp64 NumPy oracle of the PISA forward pass - TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Sources (the pages describing "PISA: Piecewise Sparse Attention Is Wiser for Efficient Diffusion
Transformers", arXiv 2602.01077):

* [gist-2] gist.science technical summary, section 2 "Method": the critical/long-tail split,
  the output as a normalised numerator over denominator, the three kinds of term, the printed
  numerator formula with alpha, the global first-order statistic H-bar, covariance-aware
  routing with M_j, and the fused-kernel phases.
* [radio] AI Radio episode on PISA, paper-summary segment: blocks of size B, the per-query
  split into S_i and U_i, the shared scale factor beta_t, the routing score Score_{t,j}.
* [abstract] the paper abstract (paperchime / mlsanity / chatpaper pages): keep-or-drop versus
  exact-or-approximate.

Readings where the pages are silent or garbled (each also listed in the design doc):

R1  softmax scale tau = 1/sqrt(d) is folded into the query everywhere (q~ = tau q): exact scores,
    alpha, the pooled routing query and the first-order term q~ H-bar.
R2  query blocks use the same block size B as key/value blocks.
R2' the denominator D_t has no first-order part: expanding exp(q~ k_n) about the block centroid
    gives the first-order sum q~ . sum_n (k_n - kbar_j), which is zero because kbar_j is the mean.
R3  "centroid" = arithmetic mean of the block's keys.
R4  block first-order matrix H_j = sum_n (k_n - kbar_j)^T v_n  (d x d; n_j times the in-block
    key/value covariance).
R5  H-bar = unweighted mean of H_j over all N_b blocks of the (batch, head), partial block included.
R6  ||.||_2 of a matrix read as the Frobenius norm (spectral norm kept as an option).
R7  routing score Score_{i,j} = qbar_i . kbar_j + ln(n_j + ||qbar_i|| M_j)  ("cov"); "plain" is
    qbar_i . kbar_j.  Ranking by alpha (n_j + ||q~|| M_j): the zeroth-order mass plus the bound on
    the first-order numerator error alpha q~ (H_j - H-bar), in logs, at the pooled query.
R8  pooled query of a query block = mean of q~ over its rows.
R9  k = clamp(ceil(keep N_b - 1e-9), 1, N_b).
R10 ties: larger score first, then smaller block index; S_i is a set.
R11 a ragged last block has n_j = L - (N_b - 1) B rows; every formula uses n_j.
R12 no forced blocks (diagonal, first, text): pure top-k.
R15 the softmax shift m_t is the max over exact scores and over a_{t,j} + ln n_j; any common
    shift gives the same ratio.
"""

from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

__all__ = [
    "n_blocks", "block_bounds", "top_k_count", "HeadStats", "head_stats", "routing_scores",
    "select_blocks", "piecewise_rows", "pisa_head", "pisa", "dense_attention", "executed_flops",
]


# ---------------------------------------------------------------------------------------------
# Block partition  ([radio] paper summary: everything is cut into blocks of size B)
# ---------------------------------------------------------------------------------------------

def n_blocks(L: int, B: int) -> int:
    """N_b = ceil(L / B)."""
    return -(-int(L) // int(B))


def block_bounds(L: int, B: int) -> List[tuple]:
    """Row ranges R_j = [jB, min(L, (j+1)B)) of every block (R11: the last may be ragged)."""
    return [(j * B, min(L, (j + 1) * B)) for j in range(n_blocks(L, B))]


def top_k_count(keep: float, nb: int) -> int:
    """Number of exactly computed blocks per query block, k (R9)."""
    return int(min(max(math.ceil(keep * nb - 1e-9), 1), nb))


# ---------------------------------------------------------------------------------------------
# Precompute: centroids, value sums, block first-order matrices, H-bar, M_j
# ([gist-2] fused-kernel precompute step; zeroth-order term; global first-order correction;
#  covariance-aware routing)
# ---------------------------------------------------------------------------------------------

@dataclasses.dataclass
class HeadStats:
    n: np.ndarray        # [Nb] rows per block n_j
    qbar: np.ndarray     # [Nb, d] pooled scaled query of each query block (R8)
    kbar: np.ndarray     # [Nb, d] key centroid (R3)
    vsum: np.ndarray     # [Nb, d] value sum  sum_n v_{j,n}
    H: np.ndarray        # [Nb, d, d] block first-order matrices (R4)
    Hbar: np.ndarray     # [d, d] mean of H_j over all blocks (R5)
    M: np.ndarray        # [Nb] ||H_j - Hbar|| (R6)


def head_stats(q: np.ndarray, k: np.ndarray, v: np.ndarray, B: int, scale: float,
               norm: str = "fro") -> HeadStats:
    """Per-head block statistics.

    Pinned by: the brute-force loops (``brute.block_stats``), the closed-form identity
    H-bar = (K^T V - sum_j n_j kbar_j vbar_j^T) / N_b, constant-key blocks giving H_j = 0, and
    B = 1 giving H_j = 0 (tests/test_oracle_pins.py).
    """
    L, d = k.shape
    bounds = block_bounds(L, B)
    nb = len(bounds)
    qt = scale * q
    n = np.array([e - s for s, e in bounds], dtype=np.float64)
    qbar = np.empty((nb, d))
    kbar = np.empty((nb, d))
    vsum = np.empty((nb, d))
    H = np.empty((nb, d, d))
    for j, (s, e) in enumerate(bounds):
        kbar[j] = k[s:e].mean(axis=0)
        vsum[j] = v[s:e].sum(axis=0)
        qbar[j] = qt[s:e].mean(axis=0)
        H[j] = (k[s:e] - kbar[j]).T @ v[s:e]
    Hbar = H.mean(axis=0)
    diff = H - Hbar
    if norm == "fro":
        M = np.sqrt(np.einsum("jab,jab->j", diff, diff))
    elif norm == "spectral":
        M = np.array([np.linalg.norm(x, ord=2) for x in diff])
    else:
        raise ValueError(norm)
    return HeadStats(n=n, qbar=qbar, kbar=kbar, vsum=vsum, H=H, Hbar=Hbar, M=M)


# ---------------------------------------------------------------------------------------------
# Routing ([gist-2] covariance-aware routing; [radio] Score_{t,j})
# ---------------------------------------------------------------------------------------------

def routing_scores(st: HeadStats, routing: str = "cov") -> np.ndarray:
    """Score_{i,j} for every (query block i, key block j), shape [Nb, Nb].

    "plain": qbar_i . kbar_j - pinned by the textbook top-k of the pooled product.
    "cov":   qbar_i . kbar_j + ln(n_j + ||qbar_i||_2 M_j)  (R7, a reading: the pages name the
             ingredients, not the formula). Each term is pinned by properties that fix it: with
             every M_j = 0 (constant keys per block, ragged last block) cov - plain = ln n_j; for
             two blocks with equal centroids the score gap is ln((n + |qbar| M_0)/(n + |qbar| M_1))
             with |qbar| and M_j formed outside the oracle; and |qbar (H_j - Hbar)| <= |qbar| M_j
             (tests/test_oracle_pins.py). The choice of formula itself stays a reading.
    """
    base = st.qbar @ st.kbar.T
    if routing == "plain":
        return base
    if routing != "cov":
        raise ValueError(routing)
    qn = np.sqrt(np.einsum("id,id->i", st.qbar, st.qbar))
    return base + np.log(st.n[None, :] + qn[:, None] * st.M[None, :])


def select_blocks(scores: np.ndarray, k: int) -> List[np.ndarray]:
    """S_i: the k best blocks of each row by (score descending, index ascending) (R10), returned
    as ascending index arrays. Pinned by brute-force sorting on tiny inputs."""
    nb = scores.shape[1]
    j = np.arange(nb)
    out = []
    for row in scores:
        order = np.lexsort((j, -row))  # last key is primary: -score, then j
        out.append(np.sort(order[:k]))
    return out


# ---------------------------------------------------------------------------------------------
# Piecewise numerator / denominator ([gist-2] core algorithm)
# ---------------------------------------------------------------------------------------------

def piecewise_rows(qt_rows: np.ndarray, k: np.ndarray, v: np.ndarray, st: HeadStats,
                   S: Sequence[int], B: int, first_order: str = "global", drop: bool = False,
                   return_parts: bool = False):
    """o_t = N_t / D_t for the query rows of one query block, given its critical set S.

    N_t = sum_{j in S} sum_n e^{s_{t,n} - m} v_n                      (exact sparse term)
        + sum_{j in U} e^{a_{t,j} - m} (sum_n v_{j,n})               (block zeroth order)
        + beta_t q~_t H-bar,   beta_t = sum_{j in U} e^{a_{t,j} - m}  (global first order)
    D_t = sum_{j in S} sum_n e^{s_{t,n} - m} + sum_{j in U} n_j e^{a_{t,j} - m}       (R2')
    with s_{t,n} = q~_t . k_n, a_{t,j} = q~_t . kbar_j (alpha_{t,j} = e^{a_{t,j}}) and the shift m_t
    of R15.

    first_order: "global" (the method), "block" (per-block H_j instead of H-bar, the variant the
    method rejects as memory-bound), "none" (zeroth order only). drop=True ignores U entirely
    (keep-or-drop block-sparse attention).
    """
    L = k.shape[0]
    bounds = block_bounds(L, B)
    nb = len(bounds)
    S = sorted(int(j) for j in S)
    in_s = np.zeros(nb, dtype=bool)
    in_s[S] = True
    U = [] if drop else [j for j in range(nb) if not in_s[j]]

    if S:
        rows = np.concatenate([np.arange(*bounds[j]) for j in S])
        s = qt_rows @ k[rows].T
        vx = v[rows]
    else:
        s = np.zeros((qt_rows.shape[0], 0))
        vx = np.zeros((0, v.shape[1]))
    a = qt_rows @ st.kbar[U].T if U else np.zeros((qt_rows.shape[0], 0))
    lnn = np.log(st.n[U]) if U else np.zeros(0)

    cand = []
    if s.shape[1]:
        cand.append(s.max(axis=1))
    if a.shape[1]:
        cand.append((a + lnn[None, :]).max(axis=1))
    m = np.max(np.stack(cand, axis=0), axis=0)

    es = np.exp(s - m[:, None])
    ea = np.exp(a - m[:, None])
    N = es @ vx
    D = es.sum(axis=1)
    if U:
        N = N + ea @ st.vsum[U]
        D = D + ea @ st.n[U]
        if first_order == "global":
            beta = ea.sum(axis=1)
            N = N + beta[:, None] * (qt_rows @ st.Hbar)
        elif first_order == "block":
            for c, j in enumerate(U):
                N = N + ea[:, c:c + 1] * (qt_rows @ st.H[j])
        elif first_order != "none":
            raise ValueError(first_order)
    out = N / D[:, None]
    if return_parts:
        return out, N, D, m
    return out


def pisa_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, B: int, keep: float,
              scale: Optional[float] = None, routing: str = "cov", first_order: str = "global",
              drop: bool = False, selection: Optional[Sequence[Sequence[int]]] = None,
              query_blocks: Optional[Sequence[int]] = None, norm: str = "fro") -> dict:
    """The whole forward pass for one (batch, head): statistics -> routing -> selection ->
    piecewise rows.

    Returns a dict with ``out`` ([L, d], rows of query blocks not requested are NaN), ``S`` (the
    selection, list of ascending index arrays), ``scores`` and ``stats``.
    ``selection`` overrides the routed S_i (R16: near-tie comparisons).
    """
    L, d = q.shape
    tau = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = head_stats(q, k, v, B, tau, norm=norm)
    nb = len(st.n)
    kk = top_k_count(keep, nb)
    scores = routing_scores(st, routing)
    S = select_blocks(scores, kk) if selection is None else [np.sort(np.asarray(s, dtype=np.int64)) for s in selection]
    bounds = block_bounds(L, B)
    qb = range(nb) if query_blocks is None else query_blocks
    out = np.full((L, d), np.nan)
    qt = tau * q
    for i in qb:
        s0, e0 = bounds[i]
        out[s0:e0] = piecewise_rows(qt[s0:e0], k, v, st, S[i], B, first_order=first_order, drop=drop)
    return {"out": out, "S": S, "scores": scores, "stats": st, "k": kk, "scale": tau}


def pisa(Q: np.ndarray, K: np.ndarray, V: np.ndarray, B: int, keep: float, **kw) -> np.ndarray:
    """Batched over heads: Q, K, V are [H, L, d] fp64; returns out [H, L, d]."""
    return np.stack([pisa_head(Q[h], K[h], V[h], B, keep, **kw)["out"] for h in range(Q.shape[0])])


# ---------------------------------------------------------------------------------------------
# Dense softmax attention: the quantity the method stands in for (quality reference)
# ---------------------------------------------------------------------------------------------

def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: Optional[float] = None,
                    rows: Optional[np.ndarray] = None) -> np.ndarray:
    """softmax(q~ K^T) V for the given query rows (all rows by default), fp64."""
    d = q.shape[1]
    tau = 1.0 / math.sqrt(d) if scale is None else float(scale)
    qq = q if rows is None else q[rows]
    s = (tau * qq) @ k.T
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return (p @ v) / p.sum(axis=1, keepdims=True)


# ---------------------------------------------------------------------------------------------
# Algorithmic FLOP count (what the method must compute, at true sizes)
# ---------------------------------------------------------------------------------------------

def executed_flops(L: int, d: int, B: int, S: Sequence[Sequence[int]]) -> dict:
    """FLOPs of one head: exact part sum_i sum_{j in S_i} 4 n_i n_j d, zeroth-order part
    sum_i 4 n_i |U_i| d, first-order part 2 L d^2, statistics 2 (2 L d^2) (K^T V formed twice:
    once for H-bar, once for M_j) and routing scores 2 N_b^2 d."""
    bounds = block_bounds(L, B)
    n = [e - s for s, e in bounds]
    nb = len(n)
    exact = 0
    zeroth = 0
    for i, Si in enumerate(S):
        exact += sum(4 * n[i] * n[j] * d for j in Si)
        zeroth += 4 * n[i] * (nb - len(Si)) * d
    first = 2 * L * d * d
    stats = 4 * L * d * d
    route = 2 * nb * nb * d
    return {"exact": exact, "zeroth": zeroth, "first": first, "stats": stats, "route": route,
            "attend": exact + zeroth + first, "total": exact + zeroth + first + stats + route}
