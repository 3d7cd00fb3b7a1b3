"""Writes tests/golden/tiny_taylor.json: a tiny ragged case (L=23, d=4, B=5, keep=0.4) with its
inputs, the routed selection and the output of the pure-Python element-loop expansion in
oracle/brute.py (the method's block-wise Taylor expansion with the global first-order term).

The pages print no operator-level worked example, so this fixture is a regression anchor for the
oracle, produced by oracle code only: run ``python tests/golden/make_golden.py`` from the repo root.
"""
import json
import math
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from oracle import brute  # noqa: E402

L, d, B, keep = 23, 4, 5, 0.4
rng = np.random.default_rng(2024)
q, k, v = (np.round(rng.standard_normal((L, d)), 3).tolist() for _ in range(3))
tau = 1 / math.sqrt(d)
st = brute.block_stats(q, k, v, B, tau)
nb = len(st["n"])
k_top = min(max(math.ceil(keep * nb - 1e-9), 1), nb)
S, scores = brute.route(st, k_top, "cov")
out = {}
for fo in ("global", "block", "none"):
    out[fo] = brute.taylor_rows(q, k, v, B, tau, S, first_order=fo)
out["drop"] = brute.taylor_rows(q, k, v, B, tau, S, drop=True)
doc = {"L": L, "d": d, "B": B, "keep": keep, "scale": tau, "q": q, "k": k, "v": v,
       "S": S, "scores": scores, "out": out,
       "source": "oracle/brute.py element loops; no printed example exists on the pages"}
path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_taylor.json")
with open(path, "w") as f:
    json.dump(doc, f, indent=1)
print("wrote", path)
