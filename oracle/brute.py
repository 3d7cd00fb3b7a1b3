"""Pure-Python element loops for tiny inputs - TEST INFRASTRUCTURE ONLY.

Written independently of ``pisa_oracle`` (no NumPy, no shared helpers) to pin it:

* ``block_stats``: centroids, value sums, H_j and H-bar by explicit sums over rows.
* ``taylor_rows``: per element, the first-order Taylor expansion of exp(q~ k_n) about the block
  centroid, exp(q~ kbar)(1 + q~ (k_n - kbar)), summed into numerator and denominator without any
  max shift ([gist-2] core algorithm: block-wise Taylor expansion of the long-tail set; with
  ``first_order="block"`` this is the expansion itself, with ``"global"`` the per-block
  first-order numerator part is replaced by the H-bar term, with ``"none"`` dropped).
* ``route``: scores and the (score desc, index asc) top-k by a full sort.
* ``spectral_norm``: largest singular value by power iteration (the spectral reading of M_j).

Inputs are lists of lists of floats (or anything indexable that yields floats).
"""

from __future__ import annotations

import math


def _blocks(L, B):
    out = []
    s = 0
    while s < L:
        out.append((s, min(L, s + B)))
        s += B
    return out


def block_stats(q, k, v, B, scale):
    L = len(k)
    d = len(k[0])
    bl = _blocks(L, B)
    kbar, vsum, qbar, H, n = [], [], [], [], []
    for (s, e) in bl:
        cnt = e - s
        n.append(cnt)
        kb = [sum(k[r][c] for r in range(s, e)) / cnt for c in range(d)]
        vs = [sum(v[r][c] for r in range(s, e)) for c in range(d)]
        qb = [sum(scale * q[r][c] for r in range(s, e)) / cnt for c in range(d)]
        Hj = [[sum((k[r][a] - kb[a]) * v[r][b] for r in range(s, e)) for b in range(d)]
              for a in range(d)]
        kbar.append(kb)
        vsum.append(vs)
        qbar.append(qb)
        H.append(Hj)
    nb = len(bl)
    Hbar = [[sum(H[j][a][b] for j in range(nb)) / nb for b in range(d)] for a in range(d)]
    M = [math.sqrt(sum((H[j][a][b] - Hbar[a][b]) ** 2 for a in range(d) for b in range(d)))
         for j in range(nb)]
    return {"n": n, "kbar": kbar, "vsum": vsum, "qbar": qbar, "H": H, "Hbar": Hbar, "M": M,
            "blocks": bl}


def spectral_norm(E, iters=4000):
    """Largest singular value of a small square matrix (list of rows) by plain power iteration on
    E^T E from the all-ones vector, then sqrt of the Rayleigh quotient."""
    d = len(E)
    x = [1.0] * d
    lam = 0.0
    for _ in range(iters):
        y = [sum(E[r][c] * x[c] for c in range(d)) for r in range(d)]      # E x
        z = [sum(E[r][c] * y[r] for r in range(d)) for c in range(d)]      # E^T E x
        nz = math.sqrt(sum(t * t for t in z))
        if nz == 0.0:
            return 0.0
        nx = math.sqrt(sum(t * t for t in x))
        lam = sum(a * b for a, b in zip(x, z)) / (nx * nx)
        x = [t / nz for t in z]
    return math.sqrt(max(lam, 0.0))


def route(st, k_top, routing="cov"):
    nb = len(st["n"])
    d = len(st["kbar"][0])
    S = []
    scores = []
    for i in range(nb):
        qb = st["qbar"][i]
        qn = math.sqrt(sum(x * x for x in qb))
        row = []
        for j in range(nb):
            sc = sum(qb[c] * st["kbar"][j][c] for c in range(d))
            if routing == "cov":
                sc += math.log(st["n"][j] + qn * st["M"][j])
            row.append(sc)
        scores.append(row)
        ranked = sorted(range(nb), key=lambda j: (-row[j], j))
        S.append(sorted(ranked[:k_top]))
    return S, scores


def taylor_rows(q, k, v, B, scale, S, first_order="global", drop=False):
    """Output rows for every token t, given S[i] per query block i."""
    L = len(q)
    d = len(q[0])
    st = block_stats(q, k, v, B, scale)
    bl = st["blocks"]
    out = []
    for i, (s0, e0) in enumerate(bl):
        sel = set(S[i])
        for t in range(s0, e0):
            qt = [scale * x for x in q[t]]
            num = [0.0] * d
            den = 0.0
            beta = 0.0
            for j, (s, e) in enumerate(bl):
                if j in sel:
                    for r in range(s, e):
                        w = math.exp(sum(qt[c] * k[r][c] for c in range(d)))
                        den += w
                        for c in range(d):
                            num[c] += w * v[r][c]
                    continue
                if drop:
                    continue
                kb = st["kbar"][j]
                alpha = math.exp(sum(qt[c] * kb[c] for c in range(d)))
                beta += alpha
                for r in range(s, e):
                    lin = sum(qt[c] * (k[r][c] - kb[c]) for c in range(d))
                    # zeroth order of the numerator and the denominator
                    den += alpha * (1.0 + lin)
                    for c in range(d):
                        num[c] += alpha * v[r][c]
                        if first_order == "block":
                            num[c] += alpha * lin * v[r][c]
            if first_order == "global" and not drop:
                for b in range(d):
                    num[b] += beta * sum(qt[a] * st["Hbar"][a][b] for a in range(d))
            out.append([x / den for x in num])
    return out
