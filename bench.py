#!/usr/bin/env python3
"""Benchmark of the PISA forward pass (libpisa) on one MI355X.

A step is one whole pass of the hot path over the workload: block statistics, routing and the
fused piecewise attention (pisa_forward_stats + pisa_forward_route + pisa_forward_attend, which
together are pisa_forward). Inputs are generated once (seeded, synthetic) and resident in HBM
before the timed region. HIP events recorded on the library's stream between the stages give the
per-stage time of every step; the attention kernel's average duration feeds the roofline.

Prints one JSON line. Default workload: the Wan2.1-14B-like 720p layer (40 heads, L = 75600,
d = 128, B = 128, keep 10%, bf16).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "PISA attn fwd ms/call + achieved TFLOP/s vs bf16 MFMA peak, Wan-720p shape"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_F32_VALU_TFLOPS = 157.3
PEAK_HBM_GBPS = 8000.0
# End-to-end generation speed-ups over dense attention that the pages report (gist.science summary
# of the PISA paper, section 4 "Experimental results"; the AI Radio episode gives the same
# figures). The pages name no hardware, and they time whole generations, not one attention layer:
# context for the bench line, not a target.
PAGES_SPEEDUPS = {"Wan2.1-14B (video, 87.5% sparsity)": 1.91, "HunyuanVideo (video)": 2.57,
                  "FLUX.1-dev (image, 85% sparsity)": 1.2}
ATTEND_SRC = os.path.join(ROOT, "sparse_attention_diffusion_pool_amd", "csrc", "attend_bf16.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attend_bf16_wan720p_traffic.json")


def source_sha(path: str) -> str:
    """Hash of the attention kernel's code (its source and dev_common.h) with comments and
    whitespace removed: a traffic record stays valid across comment edits, not across code edits."""
    import re
    files = [path, os.path.join(os.path.dirname(path), "dev_common.h")]
    h = hashlib.sha256()
    for f in files:
        text = open(f).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def algorithmic_flops(idx: np.ndarray, L: int, d: int, B: int, phases: int, first_order: int = 0) -> dict:
    """Executed FLOPs of one call from the actual selection idx [H, N_b, k]: exact part
    4 n_i n_j d per selected pair, zeroth-order part 4 n_i |U_i| d, first-order 2 L d^2 per head
    (block-wise variant: |U_i| (2 d^2 + 2 d) per query row), statistics 2 x 2 L d^2 per head
    (K^T V for H-bar and again for M_j), scores 2 N_b^2 d."""
    H, nb, kk = idx.shape
    n = np.full(nb, B, dtype=np.float64)
    n[-1] = L - (nb - 1) * B
    n_sel = n[idx].sum(axis=2)               # [H, N_b]: sum of n_j over S_i
    exact = float((4.0 * d * n[None, :] * n_sel).sum())
    tail = kk < nb and (phases & 2)
    zeroth = float(4.0 * d * (n.sum() * (nb - kk)) * H) if tail else 0.0
    first = 0.0
    if tail and (phases & 4):
        first = float(H * L * (nb - kk) * (2.0 * d * d + 2.0 * d)) if first_order else float(2.0 * L * d * d * H)
    stats = float(4.0 * L * d * d * H)
    route = float(2.0 * nb * nb * d * H)
    return {"exact": exact, "zeroth": zeroth, "first": first, "attend": exact + zeroth + first,
            "stats": stats, "route": route, "total": exact + zeroth + first + stats + route}


def dense_rows(q, k, v, rows, scale):
    """softmax(scale q K^T) V for the given rows of one head, float64 on the host (quality check)."""
    import torch
    qq = q[rows].to(torch.float64) * scale
    s = qq @ k.to(torch.float64).T
    p = torch.softmax(s, dim=1)
    return p @ v.to(torch.float64)


def cpu_baseline(w, heads, sample_note):
    """The fp64 oracle, as it stands, on a bounded sample of the workload (whole heads)."""
    from oracle import pisa_oracle as po
    from workloads import head_inputs, to_float64
    cores = len(os.sched_getaffinity(0))
    flops = 0.0
    secs = 0.0
    for h in heads:
        q, k, v = (to_float64(t) for t in head_inputs(w, h))
        t0 = time.perf_counter()
        r = po.pisa_head(q, k, v, w.B, w.keep)
        secs += time.perf_counter() - t0
        f = po.executed_flops(w.L, w.d, w.B, r["S"])
        flops += f["total"]
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": sample_note, "seconds": secs, "cpu": cpu_model()}


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), else the machine type."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


KERNELS = ("stats_qbar_bf16", "stats_pass_bf16", "stats_cov_chunk_bf16", "stats_cov_bf16", "stats_finalize", "stats_f32",
           "route_kernel", "attend_bf16", "mfma_probe", "attend_f32", "copyBuffer", "Fill")


def short_kernel(name: str) -> str:
    return next((k for k in KERNELS if k in name), name[:48])


def summarize_trace(d: str) -> None:
    """Markdown table from a rocprofv3 --kernel-trace --stats --output-format csv directory."""
    import csv
    path = next(os.path.join(r, f) for r, _, fs in os.walk(d) for f in fs if f.endswith("kernel_stats.csv"))
    rows = list(csv.DictReader(open(path)))
    print("| kernel | calls | average (us) | min (us) | max (us) | share |")
    print("|---|---|---|---|---|---|")
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        print(f"| {short_kernel(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
              f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")


# Counter passes for --summarize-counters (each within one rocprofv3 run's hardware limits:
# at most 8 SQ, 4 TCC and 2 GRBM counters), collected together with --kernel-trace.
COUNTER_PASSES = {
    "p1": "GRBM_GUI_ACTIVE SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_INSTS_VALU "
          "SQ_INSTS_LDS SQ_INSTS_SALU SQ_INSTS_VMEM",
    "p2": "GRBM_GUI_ACTIVE SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS "
          "SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_ANY TCC_HIT_sum TCC_MISS_sum",
}


def summarize_counters(d: str) -> None:
    """Per-kernel counter summary from the COUNTER_PASSES directories under d (rocprofv3 --kernel-trace
    --pmc ... over the benchmark). Counters are averaged per dispatch. GRBM_GUI_ACTIVE is summed over
    the 8 XCDs; SQ_VALU_MFMA_BUSY_CYCLES over the 1024 SIMDs; SQ_WAVE_CYCLES and the SQ wait / active
    counters count in units of 4 cycles per wave."""
    import collections
    import csv

    vals = collections.defaultdict(dict)
    durs = collections.defaultdict(list)
    for sub in COUNTER_PASSES:
        agg = collections.defaultdict(float)
        disp = collections.defaultdict(set)
        for r in csv.DictReader(open(os.path.join(d, sub, "run_counter_collection.csv"))):
            k = short_kernel(r["Kernel_Name"])
            agg[(k, r["Counter_Name"])] += float(r["Counter_Value"])
            disp[k].add(r["Dispatch_Id"])
        for (k, c), v in agg.items():
            vals[k][c] = v / len(disp[k])
        for r in csv.DictReader(open(os.path.join(d, sub, "run_kernel_trace.csv"))):
            durs[short_kernel(r["Kernel_Name"])].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    print("| kernel | ms (under counters) | shader clock (GHz) | MFMA busy (of SIMD cycles) | "
          "VALU / LDS / SALU / VMEM instr per MFMA | waves waiting (of wave time) | LDS bank conflicts "
          "(of LDS-active cycles) | L2 hit rate |")
    print("|---|---|---|---|---|---|---|---|")
    for k in ("attend_bf16", "stats_qbar_bf16", "stats_pass_bf16", "stats_cov_chunk_bf16", "stats_cov_bf16", "route_kernel",
              "stats_finalize", "mfma_probe"):
        a = vals.get(k)
        if not a or not durs.get(k):
            continue
        dur = sum(durs[k]) / len(durs[k])
        cyc = a["GRBM_GUI_ACTIVE"] / 8
        mf = a.get("SQ_INSTS_MFMA", 0.0)
        mix = ("/".join(f"{a[c] / mf:.2f}" for c in ("SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VMEM"))
               if mf > 0 else "-")
        busy = a.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (cyc * 1024)
        wait = a["SQ_WAIT_ANY"] / a["SQ_WAVE_CYCLES"] if a.get("SQ_WAVE_CYCLES") else float("nan")
        bank = a["SQ_LDS_BANK_CONFLICT"] / a["SQ_LDS_IDX_ACTIVE"] if a.get("SQ_LDS_IDX_ACTIVE") else 0.0
        hit = a["TCC_HIT_sum"] / max(a["TCC_HIT_sum"] + a["TCC_MISS_sum"], 1.0)
        print(f"| {k} | {dur * 1e3:.3f} | {cyc / dur / 1e9:.2f} | {busy:.3f} | {mix} | {wait:.3f} | {bank:.4f} | {hit:.3f} |")


def summarize_traffic(d: str, command: str) -> None:
    """HBM-side bytes per attention launch from two rocprofv3 --pmc passes (FETCH_SIZE, then
    WRITE_SIZE, KiB per dispatch) over the benchmark, each scaled by what the same counter reads for
    a 1 GiB device copy (bench.py --copy-calibration). Writes the traffic record the benchmark
    reports (valid while the attention kernel's sources are unchanged) and prints a summary."""
    import collections
    import csv

    def per_kernel(sub, counter):
        agg = collections.defaultdict(float)
        for r in csv.DictReader(open(os.path.join(d, sub, "run_counter_collection.csv"))):
            if r["Counter_Name"] == counter:
                agg[(int(r["Dispatch_Id"]), short_kernel(r["Kernel_Name"]))] += float(r["Counter_Value"])
        per = collections.defaultdict(list)
        for (_, k), v in agg.items():
            per[k].append(v * 1024.0)
        return {k: sum(v) / len(v) for k, v in per.items()}

    fetch, write = per_kernel("fetch", "FETCH_SIZE"), per_kernel("write", "WRITE_SIZE")
    cal = 1 << 30
    f_scale = cal / per_kernel("copy_fetch", "FETCH_SIZE")["copyBuffer"]
    w_scale = cal / per_kernel("copy_write", "WRITE_SIZE")["copyBuffer"]
    rec = {"kernel": "attend_bf16", "workload": "wan720p-like-L75600", "source_sha": source_sha(ATTEND_SRC),
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "fetch_bytes_per_launch": fetch["attend_bf16"] * f_scale,
           "write_bytes_per_launch": write["attend_bf16"] * w_scale,
           "command": command}
    rec["hbm_bytes_per_launch"] = rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(f"copy calibration (1 GiB device copy): FETCH_SIZE x {f_scale:.3f}, WRITE_SIZE x {w_scale:.3f}\n")
    print("| kernel | fetched GB per launch (scaled) | written GB per launch (scaled) |")
    print("|---|---|---|")
    for k in sorted(fetch, key=lambda k: -fetch[k]):
        if k in ("copyBuffer", "Fill"):
            continue
        print(f"| {k} | {fetch[k] * f_scale / 1e9:.3f} | {write.get(k, 0.0) * w_scale / 1e9:.3f} |")


def time_stages(plan, qd, kd, vd, out, stream, steps, warmup):
    """Per-step stage times (ms) of `steps` forwards after `warmup` untimed ones, HIP events on the
    library's stream: arrays stats, route, attend, step, plus the span of all timed steps."""
    import torch
    for _ in range(warmup):
        plan.forward(qd, kd, vd, out, stream)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    wall0 = time.perf_counter()
    for s in range(steps):
        ev[s][0].record(stream)
        plan.forward_stats(qd, kd, vd, stream)
        ev[s][1].record(stream)
        plan.forward_route(stream)
        ev[s][2].record(stream)
        plan.forward_attend(qd, kd, vd, out, stream)
        ev[s][3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    t = {name: np.array([ev[s][a].elapsed_time(ev[s][b]) for s in range(steps)])
         for name, a, b in (("stats", 0, 1), ("route", 1, 2), ("attend", 2, 3), ("step", 0, 3))}
    t["span"] = ev[0][0].elapsed_time(ev[steps - 1][3])
    t["wall_ms"] = wall * 1e3
    return t


def mfma_probe(dev, blocks: int = 2048, iters: int = 2000) -> dict:
    """The MFMA throughput and shader clock the chip sustains on a pure loop of the attention
    kernel's MFMA instruction (pisa_debug_mfma_probe): 8 workgroups of 4 waves per CU."""
    import torch
    from sparse_attention_diffusion_pool_amd import _lib as L
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    clk = torch.empty(blocks * 2, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()
    L.mfma_probe(out, clk, blocks, iters, stream)  # warm-up (clock ramp, code load)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    L.mfma_probe(out, clk, blocks, iters, stream)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b)
    c = clk.view(blocks, 2).cpu().numpy().astype(np.float64)
    flops = blocks * 4 * 4 * iters * 32768.0
    return {"tflops": round(flops / (ms * 1e-3) / 1e12, 1), "ms": round(ms, 4),
            "sclk_ghz": round(float(c[:, 0].sum() / c[:, 1].sum()) * 0.1, 3),
            "loop": f"{blocks} workgroups x 4 waves x {iters} x 4 independent v_mfma_f32_32x32x16_bf16"}


def selection_of(plan, info, H, dev):
    import torch
    idx = torch.empty((H, info["n_blocks"], info["k"]), dtype=torch.int32, device=dev)
    plan.debug_copy_selection(idx)
    torch.cuda.synchronize()
    return idx.cpu().numpy()


# (label, keep override (None = the workload's), phase mask, first order): the method, its
# block-wise first-order variant (every unselected block's own H_j instead of H-bar), its
# zeroth-order-only ablation, keep-or-drop block-sparse attention at the same k, and dense
# attention (every block exact) through the same kernel
MODES = (("pisa", None, 7, 0), ("block-wise first order", None, 7, 1), ("zeroth-order only", None, 3, 0),
         ("keep-or-drop", None, 1, 0), ("dense", 1.0, 1, 0))


def compare_modes(w, steps, warmup, quality_blocks=8):
    """One workload under every mode: time per forward, executed TFLOP/s, speed-up over dense
    through the same kernel, and relative L2 error against fp64 dense attention on sampled query
    blocks of the first and last head. Prints a markdown table and returns the records."""
    import torch
    from sparse_attention_diffusion_pool_amd import _lib as L
    from workloads import layer_inputs
    q, k, v = layer_inputs(w)
    dev = torch.device("cuda", 0)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    stream = torch.cuda.current_stream()
    dtype = L.DTYPE_BF16 if w.dtype == "bf16" else L.DTYPE_F32
    rng = np.random.default_rng(0)
    nb = -(-w.L // w.B)
    samples = [(h, int(i)) for h in (0, w.H - 1) for i in sorted(rng.choice(nb, size=min(quality_blocks, nb),
                                                                            replace=False))]
    refs = {}
    recs = []
    for label, keep, phases, first_order in MODES:
        kp = w.keep if keep is None else keep
        plan = L.Plan(w.L, w.H, w.d, w.B, kp, dtype=dtype, phases=phases, first_order=first_order)
        plan.attach_workspace(device=dev)
        info = plan.info()
        out = torch.empty_like(qd)
        t = time_stages(plan, qd, kd, vd, out, stream, steps, warmup)
        fl = algorithmic_flops(selection_of(plan, info, w.H, dev), w.L, w.d, w.B, phases, first_order)
        num = den = 0.0
        for h, i in samples:
            rows = np.arange(i * w.B, min(w.L, (i + 1) * w.B))
            if (h, i) not in refs:
                refs[(h, i)] = dense_rows(q[h], k[h], v[h], rows, info["scale"])
            ref = refs[(h, i)]
            got = out[h, rows[0]:rows[-1] + 1].to(torch.float64).cpu()
            num += float(((got - ref) ** 2).sum())
            den += float((ref ** 2).sum())
        ms = t["span"] / steps
        recs.append({"mode": label, "keep": kp, "k": info["k"], "phases": phases, "ms_per_call": ms,
                     "attend_ms": float(t["attend"].mean()), "stats_ms": float(t["stats"].mean()),
                     "route_ms": float(t["route"].mean()), "executed_flops": fl["total"],
                     "tflops": fl["total"] / (ms * 1e-3) / 1e12, "rel_l2_vs_dense": math.sqrt(num / den)})
        plan.destroy()
        del out
        torch.cuda.empty_cache()
    dense_ms = recs[-1]["ms_per_call"]
    print(f"workload {w.name} (H={w.H}, L={w.L}, d={w.d}, B={w.B}, {w.dtype}); {steps} timed calls after "
          f"{warmup} warm-up; quality: {len(samples)} query blocks of heads 0 and {w.H - 1} against fp64 dense\n")
    print("| mode | keep | k | ms per call | attention ms | executed TFLOP/s | speed-up vs dense | rel-L2 vs dense |")
    print("|---|---|---|---|---|---|---|---|")
    for r in recs:
        print(f"| {r['mode']} | {r['keep']:g} | {r['k']} | {r['ms_per_call']:.3f} | {r['attend_ms']:.3f} | "
              f"{r['tflops']:.1f} | {dense_ms / r['ms_per_call']:.2f}x | {r['rel_l2_vs_dense']:.4f} |")
    return recs


ROUTINGS = (("covariance-aware, Frobenius M_j", 0, 0), ("covariance-aware, spectral M_j", 0, 1),
            ("plain (pooled q . k only)", 1, 0))


def routing_quality(w, sharpen, steps, warmup, quality_blocks=8):
    """Routing variants on one workload: relative L2 error against fp64 dense attention (the method
    and keep-or-drop with each routing's own selection) and the statistics + routing time. Q is
    multiplied by `sharpen` (scores scale with it: larger values give peakier attention)."""
    import torch
    from sparse_attention_diffusion_pool_amd import _lib as L
    from workloads import layer_inputs
    q, k, v = layer_inputs(w)
    if sharpen != 1.0:
        q = (q.float() * sharpen).to(q.dtype)
    dev = torch.device("cuda", 0)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    stream = torch.cuda.current_stream()
    dtype = L.DTYPE_BF16 if w.dtype == "bf16" else L.DTYPE_F32
    rng = np.random.default_rng(0)
    nb = -(-w.L // w.B)
    samples = [(h, int(i)) for h in (0, w.H - 1) for i in sorted(rng.choice(nb, size=min(quality_blocks, nb),
                                                                            replace=False))]
    scale = 1.0 / math.sqrt(w.d)
    refs = {(h, i): dense_rows(q[h], k[h], v[h], np.arange(i * w.B, min(w.L, (i + 1) * w.B)), scale)
            for h, i in samples}
    den = sum(float((r ** 2).sum()) for r in refs.values())
    print(f"workload {w.name} (H={w.H}, L={w.L}, keep={w.keep}), Q scaled by {sharpen:g}; relative L2 "
          f"against fp64 dense attention on {len(samples)} query blocks of heads 0 and {w.H - 1}; "
          f"statistics + routing ms: mean of {steps} calls after {warmup} warm-up\n")
    print("| routing | method rel-L2 | keep-or-drop rel-L2 | statistics + routing ms |")
    print("|---|---|---|---|")
    recs = []
    for label, routing, norm in ROUTINGS:
        errs = {}
        t_sr = None
        for phases in (7, 1):
            plan = L.Plan(w.L, w.H, w.d, w.B, w.keep, dtype=dtype, phases=phases, routing=routing, norm=norm)
            plan.attach_workspace(device=dev)
            out = torch.empty_like(qd)
            t = time_stages(plan, qd, kd, vd, out, stream, steps, warmup)
            if phases == 7:
                t_sr = float((t["stats"] + t["route"]).mean())
            num = 0.0
            for (h, i), ref in refs.items():
                rows = np.arange(i * w.B, min(w.L, (i + 1) * w.B))
                got = out[h, rows[0]:rows[-1] + 1].to(torch.float64).cpu()
                num += float(((got - ref) ** 2).sum())
            errs[phases] = math.sqrt(num / den)
            plan.destroy()
            del out
        recs.append((label, errs[7], errs[1], t_sr))
        print(f"| {label} | {errs[7]:.4f} | {errs[1]:.4f} | {t_sr:.3f} |")
    return recs


SWEEP_GRIDS = ((4, 32, 32), (8, 32, 32), (16, 32, 32), (32, 32, 32))   # L = 4K, 8K, 16K, 32K
SWEEP_KEEP = (0.05, 0.1, 0.125, 0.2, 0.3, 0.5)


def latency_sweep(H, steps, warmup):
    """Forward latency of the method over sequence length and density (bf16, d = 128, B = 128,
    H heads, video-like token grids), against dense attention through the same kernel."""
    import torch
    from sparse_attention_diffusion_pool_amd import _lib as L
    from workloads import custom, layer_inputs
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    rows = []
    for grid in SWEEP_GRIDS:
        w = custom(f"sweep-{'x'.join(map(str, grid))}", H, grid, 128, 128, 0.1, "bf16")
        q, k, v = layer_inputs(w)
        qd, kd, vd = (t.to(dev) for t in (q, k, v))
        out = torch.empty_like(qd)
        res = {}
        for keep in SWEEP_KEEP + (1.0,):
            plan = L.Plan(w.L, H, 128, 128, keep, dtype=L.DTYPE_BF16, phases=1 if keep == 1.0 else 7)
            plan.attach_workspace(device=dev)
            t = time_stages(plan, qd, kd, vd, out, stream, steps, warmup)
            res[keep] = (t["span"] / steps, plan.info()["k"], float(t["attend"].mean()))
            plan.destroy()
        rows.append((w.L, res))
        print(f"[sweep] L={w.L}: " + " ".join(f"{kp:g}:{r[0]:.3f}ms" for kp, r in res.items()),
              file=sys.stderr, flush=True)
        del qd, kd, vd, out
        torch.cuda.empty_cache()
    print(f"bf16, H={H}, d=128, B=128, batch 1, video-like grids (T x 32 x 32); ms per forward "
          f"(statistics + routing + attention), mean of {steps} calls after {warmup} warm-up; in brackets "
          f"the speed-up over dense attention through the same kernel (keep = 1; attention stage only, since "
          f"dense attention needs no statistics or routing)\n")
    print("| L | dense ms | " + " | ".join(f"keep {kp:g}" for kp in SWEEP_KEEP) + " |")
    print("|---|---|" + "---|" * len(SWEEP_KEEP))
    for Lx, res in rows:
        dense = res[1.0][2]
        print(f"| {Lx} | {dense:.3f} | " + " | ".join(f"{res[kp][0]:.3f} ({dense / res[kp][0]:.2f}x, k={res[kp][1]})"
                                                     for kp in SWEEP_KEEP) + " |")
    return rows


def power_trace(w, seconds: float = 4.0) -> None:
    """Board power while the forward pass runs back to back, then dense attention of the same layer
    through the same kernel, then the MFMA probe loop (the same instruction with no data
    movement), each for about `seconds`. A thread
    samples the amdgpu hwmon power reading (power1_input, else power1_average; microwatts) every
    20 ms. Prints a markdown summary: mean and peak power per phase, the power cap, the forward's
    time per call and the probe's rate and shader clock."""
    import glob
    import threading
    import torch
    from sparse_attention_diffusion_pool_amd import _lib as L
    from workloads import layer_inputs

    hw = sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*/"))
    src = next((os.path.join(d, f) for d in hw for f in ("power1_input", "power1_average")
                if os.path.exists(os.path.join(d, f))), None)
    cap = next((os.path.join(d, "power1_cap") for d in hw if os.path.exists(os.path.join(d, "power1_cap"))), None)
    if src is None:
        print("no amdgpu hwmon power reading on this machine", file=sys.stderr)
        sys.exit(1)
    samples, stop = [], threading.Event()

    def sampler():
        t0 = time.perf_counter()
        while not stop.is_set():
            try:
                samples.append((time.perf_counter() - t0, float(open(src).read()) / 1e6))
            except (OSError, ValueError):
                pass
            time.sleep(0.02)

    q, k, v = layer_inputs(w)
    dev = torch.device("cuda", 0)
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    plan = L.Plan(w.L, w.H, w.d, w.B, w.keep, dtype=L.DTYPE_BF16 if w.dtype == "bf16" else L.DTYPE_F32)
    plan.attach_workspace(device=dev)
    out = torch.empty_like(qd)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        plan.forward(qd, kd, vd, out, stream)
    torch.cuda.synchronize()
    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    time.sleep(0.5)
    marks = {}
    t_start = time.perf_counter()
    n_fwd = 0
    marks["forward"] = [samples[-1][0] if samples else 0.0]
    while time.perf_counter() - t_start < seconds:
        for _ in range(10):
            plan.forward(qd, kd, vd, out, stream)
        n_fwd += 10
        torch.cuda.synchronize()
    fwd_ms = (time.perf_counter() - t_start) * 1e3 / n_fwd
    marks["forward"].append(samples[-1][0])
    time.sleep(1.0)
    # dense attention of the same layer through the same kernel (keep = 1, exact phase only)
    dplan = L.Plan(w.L, w.H, w.d, w.B, 1.0, dtype=L.DTYPE_BF16 if w.dtype == "bf16" else L.DTYPE_F32, phases=1)
    dplan.attach_workspace(device=dev)
    dplan.forward(qd, kd, vd, out, stream)
    torch.cuda.synchronize()
    marks["dense"] = [samples[-1][0]]
    t_start = time.perf_counter()
    n_dense = 0
    while time.perf_counter() - t_start < seconds:
        dplan.forward_attend(qd, kd, vd, out, stream)
        n_dense += 1
        torch.cuda.synchronize()
    dense_ms = (time.perf_counter() - t_start) * 1e3 / n_dense
    marks["dense"].append(samples[-1][0])
    dplan.destroy()
    time.sleep(1.0)
    marks["probe"] = [samples[-1][0]]
    t_start = time.perf_counter()
    probes = []
    while time.perf_counter() - t_start < seconds:
        probes.append(mfma_probe(dev))
    marks["probe"].append(samples[-1][0])
    time.sleep(0.3)
    stop.set()
    th.join()
    arr = np.array(samples)

    def phase(a, b, trim=0.5):  # drop the ramp at the start of the phase
        m = (arr[:, 0] >= a + trim) & (arr[:, 0] <= b)
        return arr[m, 1]

    fw, dn, pr = phase(*marks["forward"]), phase(*marks["dense"]), phase(*marks["probe"])
    idle = arr[arr[:, 0] < 0.45, 1]
    cap_w = float(open(cap).read()) / 1e6 if cap else float("nan")
    tf = float(np.mean([r["tflops"] for r in probes]))
    ghz = float(np.mean([r["sclk_ghz"] for r in probes]))
    print(f"{w.name}: power reading {src} (every 20 ms); cap {cap_w:.0f} W\n")
    print("| phase | mean W | max W | samples | rate |")
    print("|---|---|---|---|---|")
    print(f"| idle (before) | {idle.mean():.0f} | {idle.max():.0f} | {len(idle)} | |")
    print(f"| forward back to back | {fw.mean():.0f} | {fw.max():.0f} | {len(fw)} | {fwd_ms:.2f} ms per call |")
    print(f"| dense attention (keep = 1) back to back | {dn.mean():.0f} | {dn.max():.0f} | {len(dn)} | "
          f"{dense_ms:.1f} ms per call |")
    print(f"| MFMA probe back to back | {pr.mean():.0f} | {pr.max():.0f} | {len(pr)} | "
          f"{tf:.0f} TFLOP/s at {ghz:.2f} GHz ({len(probes)} runs) |")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wan720p-like-L75600", help="workload name (workloads.WORKLOADS)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-quality", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the dense-attention comparison (profiled runs: it launches the same kernel)")
    ap.add_argument("--cpu-heads", type=int, default=5)
    ap.add_argument("--phases", type=int, default=7)
    ap.add_argument("--routing", choices=("cov", "plain"), default="cov")
    ap.add_argument("--norm", choices=("fro", "spectral"), default="fro", help="matrix norm in M_j")
    ap.add_argument("--first-order", choices=("global", "block"), default="global")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (scales the HBM byte counters)")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print a markdown summary of a rocprofv3 --stats csv output directory and exit")
    ap.add_argument("--summarize-traffic", metavar="DIR",
                    help="turn the fetch/write/copy_fetch/copy_write --pmc csv directories under DIR into "
                         "the attention kernel's traffic record and exit")
    ap.add_argument("--traffic-command", default="", help="command line recorded with --summarize-traffic")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="per-kernel counter summary (MFMA busy, clock, instruction mix, waits, LDS bank "
                         "conflicts, L2 hits) from the COUNTER_PASSES rocprofv3 directories under DIR and exit")
    ap.add_argument("--print-counter-pass", metavar="NAME", help="print the counters of one pass and exit")
    ap.add_argument("--modes", action="store_true",
                    help="compare the method, its zeroth-order-only ablation, keep-or-drop and dense attention "
                         "on the workload (markdown table) and exit")
    ap.add_argument("--sweep", action="store_true",
                    help="latency over L = 4K..32K and keep 0.05..0.5 against dense (markdown table) and exit")
    ap.add_argument("--sweep-heads", type=int, default=24)
    ap.add_argument("--routing-quality", action="store_true",
                    help="compare routing variants (error vs dense, statistics + routing time) and exit")
    ap.add_argument("--sharpen", type=float, default=1.0, help="multiply Q by this factor (--routing-quality)")
    ap.add_argument("--power-trace", action="store_true",
                    help="board power while the forward pass, dense attention through the same kernel and the "
                         "MFMA probe loop each run back to back (markdown table), and exit")
    args = ap.parse_args()

    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_traffic:
        summarize_traffic(args.summarize_traffic, args.traffic_command)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.print_counter_pass:
        print(COUNTER_PASSES[args.print_counter_pass])
        return

    if args.copy_calibration:
        import torch
        n = 1 << 28
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"bytes_read": 4 * n, "bytes_written": 4 * n}}))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: libpisa runs on a single MI355X and has no multi-GPU path "
              "(heads would shard across GPUs with no exchange); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.modes:
        from workloads import workload
        compare_modes(workload(args.workload), args.steps, args.warmup)
        return
    if args.sweep:
        latency_sweep(args.sweep_heads, args.steps, args.warmup)
        return
    if args.power_trace:
        from workloads import workload
        power_trace(workload(args.workload))
        return
    if args.routing_quality:
        from workloads import workload
        routing_quality(workload(args.workload), args.sharpen, args.steps, args.warmup)
        return

    import torch
    from sparse_attention_diffusion_pool_amd import _lib as L
    from workloads import layer_inputs, workload

    w = workload(args.workload)
    t_gen = time.perf_counter()
    q, k, v = layer_inputs(w)
    t_gen = time.perf_counter() - t_gen
    dev = torch.device("cuda", 0)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    dtype = L.DTYPE_BF16 if w.dtype == "bf16" else L.DTYPE_F32
    first_order = 1 if args.first_order == "block" else 0
    plan = L.Plan(w.L, w.H, w.d, w.B, w.keep, dtype=dtype, phases=args.phases,
                  routing=1 if args.routing == "plain" else 0, norm=1 if args.norm == "spectral" else 0,
                  first_order=first_order)
    plan.attach_workspace(device=dev)
    info = plan.info()
    out = torch.empty_like(qd)
    stream = torch.cuda.current_stream()
    print(f"[bench] {w.name}: generated in {t_gen:.1f}s; N_b={info['n_blocks']} k={info['k']}", file=sys.stderr, flush=True)

    K = args.steps
    t = time_stages(plan, qd, kd, vd, out, stream, K, args.warmup)
    step_ms, stats_ms, route_ms, attend_ms = t["step"], t["stats"], t["route"], t["attend"]
    ms_per_step = t["span"] / K

    fl = algorithmic_flops(selection_of(plan, info, w.H, dev), w.L, w.d, w.B, args.phases, first_order)
    tflops = fl["total"] / (ms_per_step * 1e-3) / 1e12
    attend_tflops = fl["attend"] / (attend_ms.mean() * 1e-3) / 1e12
    stats_gbps = info["bytes_stats"] / (stats_ms.mean() * 1e-3) / 1e9
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_VALU_TFLOPS
    esize = 2 if w.dtype == "bf16" else 4

    traffic = None
    default_mode = args.phases == 7 and args.routing == "cov" and args.norm == "fro" and first_order == 0
    if os.path.exists(TRAFFIC_FILE) and w.cfg_id == 3 and default_mode:
        tr = json.load(open(TRAFFIC_FILE))
        if tr.get("source_sha") == source_sha(ATTEND_SRC):
            traffic = tr.get("hbm_bytes_per_launch")

    res = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded random-Fourier-feature Q/K of the layer's token grid, V ~ N(0,1))",
        "config": {"workload": w.name, "H": w.H, "L": w.L, "d": w.d, "B": w.B, "keep": w.keep,
                   "n_blocks": info["n_blocks"], "k": info["k"], "phases": args.phases,
                   "routing": args.routing, "norm": args.norm, "first_order": args.first_order},
        "frac_of_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "ms": {"step_median": round(float(np.median(step_ms)), 4), "step_min": round(float(step_ms.min()), 4),
               "stats": round(float(stats_ms.mean()), 4), "route": round(float(route_ms.mean()), 4),
               "attend": round(float(attend_ms.mean()), 4),
               "wall_per_step": round(t["wall_ms"] / K, 4)},
        "executed_flops": fl,
        "stats_hbm": {"bytes": info["bytes_stats"], "GBps": round(stats_gbps, 1),
                      "frac": round(stats_gbps / PEAK_HBM_GBPS, 4)},
        "roofline": {"kernel": "attend_bf16" if w.dtype == "bf16" else "attend_f32",
                     "bound": "mfma" if w.dtype == "bf16" else "alu",
                     "achieved": round(attend_tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(attend_tflops / peak, 4), "traffic": traffic,
                     # HBM-side bytes over the compulsory Q, K, V reads and out write of one launch
                     "traffic_ratio": (round(traffic / (4.0 * w.H * w.L * w.d * esize), 2)
                                       if traffic is not None else None)},
    }

    if w.dtype == "bf16" and args.phases == 7 and not args.no_context:
        # dense attention of the same layer through the same kernel (keep = 1, exact phase only)
        plan_dense = L.Plan(w.L, w.H, w.d, w.B, 1.0, dtype=dtype, phases=1)
        plan_dense.attach_workspace(device=dev)
        out_dense = torch.empty_like(qd)
        td = time_stages(plan_dense, qd, kd, vd, out_dense, stream, 3, 1)
        dense_ms = float(td["attend"].mean())
        res["context"] = {"pages_end_to_end_speedups": PAGES_SPEEDUPS, "pages_hardware": "not named",
                          "dense_attention_ms": round(dense_ms, 3),
                          "speedup_vs_dense_attention": round(dense_ms / ms_per_step, 2),
                          "note": "this layer's whole call against dense attention of the same layer "
                                  "through the same kernel; the pages' figures are whole generations"}
        plan_dense.destroy()
        del out_dense

    if w.dtype == "bf16":
        # measured MFMA ceiling on this machine, beside the spec peak of the roofline object
        mp = mfma_probe(dev)
        mp["attend_frac"] = round(attend_tflops / mp["tflops"], 4)
        res["mfma_probe"] = mp

    if not args.no_quality:
        # quality check on sampled query blocks of 2 heads: relative L2 of PISA (this run's output)
        # and of keep-or-drop (same kernel, exact phase only) against dense softmax attention
        plan_drop = L.Plan(w.L, w.H, w.d, w.B, w.keep, dtype=dtype, phases=1)
        plan_drop.attach_workspace(device=dev)
        out_drop = torch.empty_like(qd)
        plan_drop.forward(qd, kd, vd, out_drop, stream)
        torch.cuda.synchronize()
        rng = np.random.default_rng(0)
        nb = info["n_blocks"]
        num = {"pisa": 0.0, "drop": 0.0}
        den = 0.0
        for h in (0, w.H - 1):
            for i in sorted(rng.choice(nb, size=min(8, nb), replace=False)):
                rows = np.arange(i * w.B, min(w.L, (i + 1) * w.B))
                ref = dense_rows(q[h], k[h], v[h], rows, info["scale"])
                den += float((ref ** 2).sum())
                for name, o in (("pisa", out), ("drop", out_drop)):
                    got = o[h, rows[0]:rows[-1] + 1].to(torch.float64).cpu()
                    num[name] += float(((got - ref) ** 2).sum())
        res["quality"] = {"rel_l2_vs_dense": {"pisa": math.sqrt(num["pisa"] / den),
                                              "keep_or_drop": math.sqrt(num["drop"] / den)},
                          "sample": "16 query blocks (8 random in the first and last head), dense fp64"}
        plan_drop.destroy()

    if not args.no_cpu_baseline:
        heads = list(range(min(args.cpu_heads, w.H)))
        note = (f"{len(heads)} of {w.H} heads of {w.name}, every query block: statistics, routing, "
                f"piecewise rows (NumPy fp64); TFLOP/s of the same executed-FLOP count")
        res["cpu_baseline"] = cpu_baseline(w, heads, note)

    plan.destroy()
    print(json.dumps(res))


if __name__ == "__main__":
    main()
