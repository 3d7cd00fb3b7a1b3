"""Planted mistakes in the fp64 oracle, used to check that its pins catch them (CPU only).

Each mutant replaces one function of ``oracle.pisa_oracle`` in the running process with a copy
that carries one plausible error (a dropped term, a wrong sign, index or normalisation, a
transposed operand). ``tests/test_oracle_mutations.py`` runs the pin suite in a subprocess with
``PISA_ORACLE_MUTANT=<name>`` (applied by ``tests/conftest.py``) and requires it to fail. The oracle
file itself is never modified.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np


def _recompute_m(st, Hbar=None, H=None):
    H = st.H if H is None else H
    Hbar = st.Hbar if Hbar is None else Hbar
    diff = H - Hbar
    return np.sqrt(np.einsum("jab,jab->j", diff, diff))


def _wrap_stats(po, edit):
    orig = po.head_stats

    def head_stats(q, k, v, B, scale, norm="fro"):
        return edit(orig(q, k, v, B, scale, norm=norm), q, k, v, B, scale)

    po.head_stats = head_stats


def _wrap_rows(po, edit):
    orig = po.piecewise_rows

    def piecewise_rows(qt_rows, k, v, st, S, B, first_order="global", drop=False, return_parts=False):
        args = edit(dict(qt_rows=qt_rows, k=k, v=v, st=st, S=S, B=B, first_order=first_order, drop=drop,
                         return_parts=return_parts))
        return orig(**args)

    po.piecewise_rows = piecewise_rows


def no_first_order(po):
    """The global first-order correction is left out of the numerator."""
    _wrap_rows(po, lambda a: {**a, "first_order": "none" if a["first_order"] == "global" else a["first_order"]})


def hbar_transposed(po):
    """H-bar used transposed (q~ H-bar^T)."""
    _wrap_stats(po, lambda st, *_: dataclasses.replace(st, Hbar=st.Hbar.T.copy()))


def hbar_summed(po):
    """H-bar as the sum of the H_j instead of their mean (M_j follows it)."""
    def edit(st, *_):
        hb = st.Hbar * len(st.n)
        return dataclasses.replace(st, Hbar=hb, M=_recompute_m(st, Hbar=hb))
    _wrap_stats(po, edit)


def h_not_centred(po):
    """H_j = K_j^T V_j without subtracting the centroid."""
    def edit(st, q, k, v, B, scale):
        H = np.stack([k[s:e].T @ v[s:e] for s, e in po.block_bounds(len(k), B)])
        hb = H.mean(axis=0)
        return dataclasses.replace(st, H=H, Hbar=hb, M=_recompute_m(st, Hbar=hb, H=H))
    _wrap_stats(po, edit)


def m_not_centred(po):
    """M_j = ||H_j|| instead of ||H_j - H-bar||."""
    _wrap_stats(po, lambda st, *_: dataclasses.replace(st, M=_recompute_m(st, Hbar=np.zeros_like(st.Hbar))))


def qbar_unscaled(po):
    """Pooled query without the softmax scale."""
    _wrap_stats(po, lambda st, q, k, v, B, scale: dataclasses.replace(st, qbar=st.qbar / scale))


def vmean_for_vsum(po):
    """The zeroth-order numerator uses the mean value instead of the value sum."""
    _wrap_stats(po, lambda st, *_: dataclasses.replace(st, vsum=st.vsum / st.n[:, None]))


def ragged_counted_full(po):
    """The ragged last block counted as a full block of B rows (n_j = B everywhere)."""
    def edit(st, q, k, v, B, scale):
        return dataclasses.replace(st, n=np.full_like(st.n, float(B)))
    _wrap_stats(po, edit)


def denominator_without_counts(po):
    """Zeroth-order denominator sums alpha instead of n_j alpha."""
    _wrap_rows(po, lambda a: {**a, "st": dataclasses.replace(a["st"], n=np.ones_like(a["st"].n))})


def exact_scores_unscaled(po):
    """Exact, pooled and first-order terms use the unscaled query."""
    _wrap_rows(po, lambda a: {**a, "qt_rows": a["qt_rows"] * math.sqrt(a["k"].shape[1])})


def routing_sign(po):
    """Routing keeps the lowest scores."""
    orig = po.routing_scores
    po.routing_scores = lambda st, routing="cov": -orig(st, routing)


def routing_no_log(po):
    """Covariance-aware score adds n_j + |qbar| M_j without the logarithm."""
    orig = po.routing_scores

    def routing_scores(st, routing="cov"):
        if routing != "cov":
            return orig(st, routing)
        qn = np.sqrt(np.einsum("id,id->i", st.qbar, st.qbar))
        return st.qbar @ st.kbar.T + st.n[None, :] + qn[:, None] * st.M[None, :]

    po.routing_scores = routing_scores


def _cov_term_mutant(po, term):
    orig = po.routing_scores

    def routing_scores(st, routing="cov"):
        if routing != "cov":
            return orig(st, routing)
        qn = np.sqrt(np.einsum("id,id->i", st.qbar, st.qbar))
        return st.qbar @ st.kbar.T + term(st.n[None, :], qn[:, None], st.M[None, :], st.qbar.shape[1])

    po.routing_scores = routing_scores


def routing_qnorm_unscaled(po):
    """Covariance term weighted by the norm of the unscaled pooled query (softmax scale 1/sqrt(d))."""
    _cov_term_mutant(po, lambda n, qn, M, d: np.log(n + qn * math.sqrt(d) * M))


def routing_no_count(po):
    """Covariance term without the block's row count: ln(|qbar| M_j)."""
    _cov_term_mutant(po, lambda n, qn, M, d: np.log(qn * M))


def routing_no_qnorm(po):
    """Covariance term without the pooled-query weight: ln(n_j + M_j)."""
    _cov_term_mutant(po, lambda n, qn, M, d: np.log(n + M))


def ties_to_higher_index(po):
    """Equal scores broken towards the larger block index."""
    def select_blocks(scores, k):
        j = np.arange(scores.shape[1])
        return [np.sort(np.lexsort((-j, -row))[:k]) for row in scores]
    po.select_blocks = select_blocks


def k_rounded_down(po):
    """k = floor(keep N_b) instead of the ceiling."""
    po.top_k_count = lambda keep, nb: int(min(max(math.floor(keep * nb), 1), nb))


def last_block_short(po):
    """The ragged last block loses its final row."""
    orig = po.block_bounds

    def block_bounds(L, B):
        b = orig(L, B)
        s, e = b[-1]
        if L % B:
            b[-1] = (s, max(s + 1, e - 1))
        return b

    po.block_bounds = block_bounds


MUTANTS = {f.__name__: f for f in (
    no_first_order, hbar_transposed, hbar_summed, h_not_centred, m_not_centred, qbar_unscaled,
    vmean_for_vsum, ragged_counted_full, denominator_without_counts, exact_scores_unscaled,
    routing_sign, routing_no_log, routing_qnorm_unscaled, routing_no_count, routing_no_qnorm,
    ties_to_higher_index, k_rounded_down, last_block_short)}


def apply(name: str) -> None:
    from oracle import pisa_oracle as po
    MUTANTS[name](po)
