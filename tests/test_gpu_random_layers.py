"""GPU parity on seeded random layer shapes (through the C ABI).

The fixed cases elsewhere are chosen by hand; these draw the shape, the block size, the density,
the phase mask and the routing at random (a fixed seed per case), so that ragged tails, chunk
boundaries of the statistics passes, pooled-tile counts and selection sizes fall where nobody
placed them. Every head's statistics and selection, and every output row, are compared with the
fp64 oracle at the usual bars (selection set-equal except near-ties; bf16 outputs max-abs 2e-2
and relative L2 5e-3; fp32 outputs max-abs 1e-5).
"""

import numpy as np
import pytest

from pisa_cases import assert_close, check_stats, compare_rows, gpu_run, log, oracle_head
from workloads import custom

pytestmark = pytest.mark.gpu


def _case(seed: int):
    rng = np.random.default_rng(1000 + seed)
    ndim = int(rng.integers(1, 4))
    target = int(rng.integers(150, 6000))
    side = max(2, int(round(target ** (1.0 / ndim))))
    grid = tuple(int(max(2, side + rng.integers(-side // 3, side // 3 + 1))) for _ in range(ndim))
    n_text = int(rng.choice([0, 0, int(rng.integers(1, 300))]))
    B = int(rng.choice([64, 128]))
    keep = float(rng.uniform(0.02, 0.6))
    phases = int(rng.choice([7, 7, 3, 1]))
    routing = int(rng.choice([0, 0, 1]))
    H = int(rng.integers(1, 4))
    dtype = "f32" if seed % 4 == 3 else "bf16"
    d = int(rng.choice([64, 128])) if dtype == "f32" else 128
    return dict(grid=grid, n_text=n_text, B=B, keep=keep, phases=phases, routing=routing, H=H, dtype=dtype, d=d)


SEEDS = list(range(8))


@pytest.mark.parametrize("seed", SEEDS)
def test_random_layer(seed):
    c = _case(seed)
    w = custom(f"random-{seed}", c["H"], c["grid"], c["d"], c["B"], c["keep"], c["dtype"], n_text=c["n_text"],
               seed=500 + seed)
    res = gpu_run(w, routing=c["routing"], phases=c["phases"], want_stats=True)
    info = res["info"]
    log(f"[random] seed {seed}: {c} -> L={w.L} N_b={info['n_blocks']} k={info['k']}")
    pairs = []
    for h in range(c["H"]):
        ref, out_ref, nsel = oracle_head(res, h)
        check_stats(res, h, ref)
        pairs.append(compare_rows(res, h, out_ref, range(len(ref["S"])), res["B"]))
        if nsel:
            log(f"[parity] random-{seed} head {h}: {nsel} rows differ by near-ties only")
    assert_close(pairs, res["dtype"], f"random-{seed}")


# The routing kernel is instantiated per count of 64-key tiles (2, 4, 6, 8, 10, 12, 16, 32, 128).
# The configurations reach 2, 4, 10 and 16, the large-N_b cases 32 and 128; these layers reach
# the others: statistics and selection of every row, outputs on sampled query blocks.
TILE_CASES = [  # (N_b, B)
    (350, 128),   # 6 tiles
    (449, 128),   # 8 tiles
    (700, 128),   # 12 tiles
    (330, 64),    # 6 tiles at B = 64
]


@pytest.mark.parametrize("nb,B", TILE_CASES, ids=[f"nb{nb}-B{B}" for nb, B in TILE_CASES])
def test_routing_tile_counts(nb, B):
    L = nb * B - 37  # ragged last block
    w = custom(f"tiles-nb{nb}-B{B}", 1, (L,), 128, B, 0.1, "bf16", seed=900 + nb)
    res = gpu_run(w, want_stats=True)
    info = res["info"]
    assert info["n_blocks"] == nb
    rng = np.random.default_rng(nb)
    qb = sorted(set(rng.choice(nb, size=6, replace=False).tolist()) | {nb - 1})
    ref, out_ref, nsel = oracle_head(res, 0, query_blocks=qb)
    check_stats(res, 0, ref)
    log(f"[parity] tiles nb={nb} B={B}: k={info['k']}, {nsel} rows differ by near-ties only")
    assert_close([compare_rows(res, 0, out_ref, qb, B)], res["dtype"], f"tiles nb={nb} B={B}")


# The bf16 statistics passes give each workgroup a range of about four consecutive (head, block)
# pairs on layers this small, so with one, two or six blocks per head a range meets two, three or
# four heads, and its partial sums of H-bar and of the centroids go to one slot per head met.
MANY_HEADS = [  # (H, L, B)
    (7, 100, 128),   # N_b = 1
    (5, 200, 128),   # N_b = 2
    (9, 330, 64),    # N_b = 6
]


@pytest.mark.parametrize("H,L,B", MANY_HEADS, ids=[f"H{H}-L{L}-B{B}" for H, L, B in MANY_HEADS])
def test_ranges_across_heads(H, L, B):
    w = custom(f"heads-H{H}-L{L}-B{B}", H, (L,), 128, B, 0.4, "bf16", seed=700 + H)
    res = gpu_run(w, want_stats=True)
    pairs = []
    for h in range(H):
        ref, out_ref, nsel = oracle_head(res, h)
        check_stats(res, h, ref)
        pairs.append(compare_rows(res, h, out_ref, range(len(ref["S"])), B))
    assert_close(pairs, res["dtype"], f"ranges across heads H={H} L={L} B={B}")
