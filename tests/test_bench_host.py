"""Host-side checks of bench.py (CPU only): the executed-FLOP model behind the roofline against
the oracle's own count, the traffic record's source hash, the profile summaries, and the refusal
to run on more than one GPU."""

import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from oracle import pisa_oracle as po  # noqa: E402


@pytest.mark.parametrize("L,B,keep,H", [(1000, 128, 0.3, 2), (4608, 64, 0.25, 3), (75600, 128, 0.1, 1),
                                        (130, 64, 0.5, 1)])
def test_flop_model_matches_the_oracle_count(L, B, keep, H):
    d = 128
    nb = po.n_blocks(L, B)
    kk = po.top_k_count(keep, nb)
    rng = np.random.default_rng(L + B)
    idx = np.stack([np.stack([np.sort(rng.choice(nb, size=kk, replace=False)) for _ in range(nb)])
                    for _ in range(H)])
    got = bench.algorithmic_flops(idx, L, d, B, phases=7)
    want = {key: 0.0 for key in ("exact", "zeroth", "first", "stats", "route")}
    for h in range(H):
        f = po.executed_flops(L, d, B, [list(r) for r in idx[h]])
        for key in want:
            want[key] += f[key]
    if kk == nb:  # no unselected blocks: no zeroth- or first-order work
        want["zeroth"] = want["first"] = 0.0
    for key, value in want.items():
        assert got[key] == pytest.approx(value, rel=1e-12), key
    assert got["attend"] == pytest.approx(want["exact"] + want["zeroth"] + want["first"], rel=1e-12)


def test_flop_model_phase_masks():
    L, B, d = 1000, 128, 128
    nb = po.n_blocks(L, B)
    idx = np.array([[[0, 3]] * nb])
    full = bench.algorithmic_flops(idx, L, d, B, phases=7)
    drop = bench.algorithmic_flops(idx, L, d, B, phases=1)
    zeroth_only = bench.algorithmic_flops(idx, L, d, B, phases=3)
    assert drop["zeroth"] == drop["first"] == 0.0 and drop["exact"] == full["exact"]
    assert zeroth_only["first"] == 0.0 and zeroth_only["zeroth"] == full["zeroth"]


def test_source_hash_ignores_comments_not_code(tmp_path):
    src = tmp_path / "k.hip"
    common = tmp_path / "dev_common.h"
    src.write_text("int f(int x) { return x + 1; }  // one\n/* block */\n")
    common.write_text("// header\nint g();\n")
    h0 = bench.source_sha(str(src))
    src.write_text("// changed comment\nint f(int x) {\n  return x + 1;\n}\n")
    assert bench.source_sha(str(src)) == h0
    src.write_text("int f(int x) { return x + 2; }\n")
    assert bench.source_sha(str(src)) != h0


def test_trace_summary(tmp_path, capsys):
    (tmp_path / "run_kernel_stats.csv").write_text(
        '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs"\n'
        '"void pisa::attend_bf16<128>(...)",7,70000,10000,90.0,9000,12000\n'
        '"stats_qbar_bf16",7,7000,1000,10.0,900,1100\n')
    bench.summarize_trace(str(tmp_path))
    out = capsys.readouterr().out.splitlines()
    assert out[2].startswith("| attend_bf16 | 7 | 10.0 | 9.0 | 12.0 | 90.0% |")
    assert out[3].startswith("| stats_qbar_bf16 | 7 | 1.0 |")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
