"""GPU parity where the softmax is sharp (through the C ABI).

The generated layers keep q.k/sqrt(d) at a standard deviation of about 1-1.5. These cases push
the attention kernel where its numerics are tested hardest:

* Q multiplied by 3 and by 6 (score spreads of about 3-4.5 and 6-9): the score rounding budget.
* Layers built so that, for some query rows, a key block processed after the first step, or a
  pooled token of an unselected block, raises the row's running maximum far above what came
  before: by about 2^18 (probabilities far above 1 against the reference in use), and by more
  than 2^40 (the online softmax must move its reference and rescale numerator, denominator and
  beta mid-stream). One softmax runs across the exact phase, the zeroth-order scan and the
  first-order correction (gist.science summary, section 2 "Hardware implementation"). The host
  checks from the oracle's scores, in the order the kernel visits keys, that such rows exist.
* A layer whose scores all sit near -60 (natural log units): against a reference of 0 every
  probability would vanish, so the reference must move down to the row maximum.

Bars as everywhere: max-abs 2e-2 and relative L2 5e-3 against the fp64 oracle run on the GPU's
own selection (bf16 inputs).
"""

import math

import numpy as np
import pytest
import torch

from oracle import pisa_oracle as po
from pisa_cases import assert_close, compare_rows, gpu_run, log, oracle_head
from workloads import custom, layer_inputs, to_float64

pytestmark = pytest.mark.gpu

STEP = 64  # keys per step of the attention kernel, exact and pooled alike


def _check_all(res, label):
    pairs = []
    for h in range(res["out"].shape[0]):
        ref, out_ref, nsel = oracle_head(res, h)
        pairs.append(compare_rows(res, h, out_ref, range(len(ref["S"])), res["B"]))
        if nsel:
            log(f"[parity] {label} head {h}: {nsel} rows differ by near-ties only")
    return assert_close(pairs, res["dtype"], label)


@pytest.mark.parametrize("B", [128, 64])
@pytest.mark.parametrize("factor", [3.0, 6.0])
def test_sharper_scores(factor, B):
    w = custom("bf16-ragged-3d", 2, (7, 11, 13), 128, B, 0.3, "bf16")
    q, k, v = layer_inputs(w)
    q = (q.to(torch.float32) * factor).to(torch.bfloat16)
    qt = to_float64(q[0]) / math.sqrt(128)
    s = qt[:512] @ to_float64(k[0]).T
    log(f"[sharp] Q x {factor}: std of q.k/sqrt(d) = {s.std():.2f}")
    res = gpu_run(w, inputs=(q, k, v))
    _check_all(res, f"Q x {factor} B={B}")


def _sharp_layer(B, seed, a=12.0):
    """One head, L = 1445 (ragged last block), d = 128, in bf16. Base Q, K ~ 0.3 N(0,1), V ~ N(0,1).
    Key block N_b - 2 is shifted by a u and query blocks 0, 1 by a u: those rows find their largest
    scores (a^2 / sqrt(d) nats above the rest: 12.7 for a = 12, 30 for a = 18.5) in a block that
    follows their other selected blocks. Key block N_b - 3 is shifted by a w; in query blocks 2 and
    3, 40 % of the rows carry +a w and 60 % carry -a w, so the block's pooled score is low and it
    stays unselected, while the +w rows find their largest score in its pooled token."""
    L, d = 1445, 128
    nb = -(-L // B)
    rng = np.random.default_rng(seed)
    q = 0.3 * rng.standard_normal((L, d))
    k = 0.3 * rng.standard_normal((L, d))
    v = rng.standard_normal((L, d))
    u, w = np.linalg.qr(rng.standard_normal((d, 2)))[0].T
    rows = lambda j: slice(j * B, min(L, (j + 1) * B))  # noqa: E731
    k[rows(nb - 2)] += a * u
    k[rows(nb - 3)] += a * w
    for i in (0, 1):
        q[rows(i)] += a * u
    for i in (2, 3):
        r = np.arange(L)[rows(i)]
        cut = r[0] + int(0.4 * len(r))
        q[r[0]:cut] += a * w
        q[cut:r[-1] + 1] -= a * w
    t = lambda x: torch.from_numpy(x[None]).to(torch.bfloat16)  # noqa: E731
    return t(q), t(k), t(v)


def _step_maxima(qt, k, st, S, B):
    """Per query row: the maximum score (natural log units, pooled tokens with their ln n_j bias)
    of each step, in the order the kernel visits keys: the selected blocks' rows in ascending block
    order, STEP keys per step; then the pooled tokens j = 0 .. N_b - 1 of the unselected blocks in
    tiles of STEP tokens."""
    L = k.shape[0]
    nb = len(st.n)
    steps = []
    for j in S:
        r0, r1 = j * B, min(L, (j + 1) * B)
        for a in range(r0, r1, STEP):
            steps.append(("exact", (qt @ k[a:min(r1, a + STEP)].T).max(axis=1)))
    sel = set(int(j) for j in S)
    pooled = qt @ st.kbar.T + np.log(st.n)[None, :]
    pooled[:, sorted(sel)] = -np.inf
    for a in range(0, nb, STEP):
        steps.append(("pooled", pooled[:, a:a + STEP].max(axis=1)))
    return steps


# (shift a, required raise in log2 units): a raise past 2^9 with probabilities kept against the
# old reference, and one past 2^40 that forces the reference to move
RAISES = [(12.0, 9), (18.5, 40)]


@pytest.mark.parametrize("a,raise_log2", RAISES, ids=["raise-2^9", "raise-2^40"])
@pytest.mark.parametrize("B", [128, 64])
def test_running_max_rescaled_mid_stream(B, a, raise_log2):
    q, k, v = _sharp_layer(B, seed=100 + B, a=a)
    L = q.shape[1]
    w = custom(f"bf16-sharp-B{B}", 1, (L,), 128, B, 0.3, "bf16")
    res = gpu_run(w, inputs=(q, k, v))
    ref, _, _ = oracle_head(res, 0, query_blocks=[])
    st = ref["stats"]
    qt = to_float64(q[0]) * ref["scale"]
    kf = to_float64(k[0])
    # rows whose maximum grows by more than 2^raise_log2 after the first step, with numerator and
    # denominator already non-zero
    margin = raise_log2 * math.log(2.0)
    n_exact = n_pooled = 0
    for i, S in enumerate(res["idx"][0]):
        steps = _step_maxima(qt[i * B:min(L, (i + 1) * B)], kf, st, [int(j) for j in S], B)
        first = steps[0][1]
        exact_max = np.max(np.stack([m for kind, m in steps if kind == "exact"]), axis=0)
        later_exact = np.max(np.stack([m for kind, m in steps[1:] if kind == "exact"] or [first * 0 - np.inf]), axis=0)
        pooled_max = np.max(np.stack([m for kind, m in steps if kind == "pooled"]), axis=0)
        n_exact += int(np.sum(later_exact > first + margin))
        n_pooled += int(np.sum(pooled_max > exact_max + margin))
    log(f"[sharp] B={B} a={a}: {n_exact} rows raise their max > 2^{raise_log2} in a later exact step, "
        f"{n_pooled} rows in a pooled step")
    assert n_exact >= B and n_pooled >= B // 4
    _check_all(res, f"running max raised mid-stream B={B} a={a}")


@pytest.mark.parametrize("B", [128, 64])
def test_uniformly_low_scores(B):
    # every key carries +26 u and every query -26 u: all scores sit near -26^2/sqrt(128) = -60 nats
    # (spread by the 0.3 N(0,1) base), so exp of a score against a reference of 0 underflows
    L, d = 1445, 128
    rng = np.random.default_rng(300 + B)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    q = 0.3 * rng.standard_normal((L, d)) - 26.0 * u
    k = 0.3 * rng.standard_normal((L, d)) + 26.0 * u
    v = rng.standard_normal((L, d))
    t = lambda x: torch.from_numpy(x[None]).to(torch.bfloat16)  # noqa: E731
    q, k, v = t(q), t(k), t(v)
    s = (to_float64(q[0][:256]) / math.sqrt(d)) @ to_float64(k[0]).T
    log(f"[sharp] low scores: max {s.max():.1f}, min {s.min():.1f} (nats)")
    assert s.max() < -45
    w = custom(f"bf16-low-B{B}", 1, (L,), 128, B, 0.3, "bf16")
    res = gpu_run(w, inputs=(q, k, v))
    _check_all(res, f"uniformly low scores B={B}")
