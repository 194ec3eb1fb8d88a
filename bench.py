#!/usr/bin/env python3
"""Benchmark of the Conv1D(width 4) -> RG-LRU forward on one MI355X.

Workload: the RecurrentGemma-2B-shaped recurrent layer, B=8, T=2048, D=2560, 10 heads of 256,
bf16 x/y, fp32 state, seeded synthetic inputs (no dataset is involved). One step = one full
rglru_forward (gate projections on MFMA, then the fused conv + gate + scan) over one batch, with
the inputs already resident in HBM. Three independent input/output sets are rotated so that a
step never re-reads the previous step's data out of the 256 MB last-level cache.

Prints ONE JSON line: throughput (tokens*channels/s) and ms/step of the whole forward, a roofline
record for the dominant kernel (its algorithmic HBM bytes per launch over its average duration,
timed with HIP events on the stream the library launches on), and the fp64 CPU oracle timed on
the host cores as a baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
METRIC = "RG-LRU fwd tokens·channels/s + % HBM peak, B=8 T=2048 D=2560 bf16"
KERNEL_SOURCES = ["rglru_device.h", "rglru_mfma.h", "rglru_gates.hip", "rglru_scan.hip",
                  "rglru_fused.hip"]
BACKWARD_SOURCES = ["rglru_device.h", "rglru_mfma.h", "rglru_backward.hip", "rglru_bwd_tiles.hip",
                    "rglru_bwd_fused.hip", "rglru_gates.hip"]
# kernels of one rglru_backward call (name prefixes in rocprofv3 output; the split-operand gate
# kernels only: the forward plans run the same kernels with a single bf16 operand)
BACKWARD_KERNELS = ["tile_bwd", "tile_preacts<256, true>", "gates_mfma<256, true>", "bwd_summary", "bwd_carry",
                    "bwd_emit", "wt_prep", "tile_dxc", "dxc_mfma", "dxc_valu", "conv_bwd", "dw_mfma",
                    "dw_valu", "colsum"]


def is_backward_kernel(name: str) -> bool:
    n = name.replace("void ", "").replace("rglru::", "")
    return any(n.startswith(k) for k in BACKWARD_KERNELS)


def is_fused_kernel(name: str) -> bool:
    """The fused forward's kernels (its main kernel and the look-back reset), not the same
    kernel's instantiation that serves the chunked plan's one-pass scan (template flag true)."""
    return ("fused_forward" in name and ", true>" not in name) or "fused_reset" in name


def kernel_source_hash(sources=None) -> str:
    h = hashlib.sha256()
    for f in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, "gated_linear_recurrence_conv1d_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str, key="hbm_bytes_per_launch", sources=None):
    """HBM bytes per launch (or per call) from a committed rocprofv3 counter summary, if it was
    taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_hash") != kernel_source_hash(sources):
        return None
    try:
        return float(vals[key])
    except (KeyError, ValueError):
        return None


# Two counter passes (rocprofv3 collects one pass per run: at most 8 SQ counters each).
PMC_PASSES = (
    ["SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES",
     "SQ_ACTIVE_INST_VALU", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "GRBM_GUI_ACTIVE"],
    ["SQ_INSTS_VALU_TRANS_F32", "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_ANY",
     "SQ_WAIT_ANY", "SQ_ACTIVE_INST_ANY", "SQ_WAVE_CYCLES", "SQ_INSTS_VALU", "GRBM_GUI_ACTIVE"],
)
# VALU issue model (cycles of one SIMD): a full-rate wave64 operation takes 2 cycles (32 lanes per
# cycle: 157.3 TFLOP/s fp32 = 256 CUs x 4 SIMDs x 2.4 GHz x 32 lanes x 2 flops per FMA), a
# transcendental (exp2, rcp, sqrt, rsq, log) a quarter of that rate, 8 cycles (measured).
VALU_CYCLES, TRANS_CYCLES, SIMDS, CLOCK_GHZ, XCDS = 2.0, 8.0, 1024, 2.4, 8

PROFILE_CMDS = {
    "trace": "rocprofv3 --kernel-trace --stats -d OUT/trace -o bench --output-format csv -- "
             "python3 REPO/bench.py --no-cpu-baseline --no-plan-legs",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --kernel-include-regex 'fused_forward|copyBuffer' -d "
             "OUT/fetch -o fetch --output-format csv -- python3 REPO/bench.py --steps 5 "
             "--warmup 5 --no-cpu-baseline --settle-s 0 --no-decode --no-backward --no-mqa --no-plan-legs "
             "--copy-calibration 256",
    "write": "rocprofv3 --pmc WRITE_SIZE --kernel-include-regex 'fused_forward|copyBuffer' -d "
             "OUT/write -o write --output-format csv -- python3 REPO/bench.py --steps 5 "
             "--warmup 5 --no-cpu-baseline --settle-s 0 --no-decode --no-backward --no-mqa --no-plan-legs "
             "--copy-calibration 256",
    "bwd_fetch": "rocprofv3 --pmc FETCH_SIZE --kernel-include-regex "
                 "'tile_|bwd_|wt_prep|dxc_|conv_bwd|dw_|colsum|copyBuffer' -d OUT/bfetch -o fetch "
                 "--output-format csv -- python3 REPO/bench.py --steps 5 --warmup 5 "
                 "--no-cpu-baseline --settle-s 0 --no-decode --no-mqa --no-plan-legs --bwd-warmup 2 "
                 "--bwd-reps 3 --copy-calibration 256",
    "bwd_write": "rocprofv3 --pmc WRITE_SIZE --kernel-include-regex "
                 "'tile_|bwd_|wt_prep|dxc_|conv_bwd|dw_|colsum|copyBuffer' -d OUT/bwrite -o write "
                 "--output-format csv -- python3 REPO/bench.py --steps 5 --warmup 5 "
                 "--no-cpu-baseline --settle-s 0 --no-decode --no-mqa --no-plan-legs --bwd-warmup 2 "
                 "--bwd-reps 3 --copy-calibration 256",
    "leg_trace": "rocprofv3 --kernel-trace --stats -d OUT/trace_W -o bench --output-format csv -- "
                 "python3 REPO/bench.py --workload W --steps 20 --warmup 10 --no-cpu-baseline "
                 "--no-backward --no-decode --no-mqa --no-plan-legs",
    "bwd_pmc1": "rocprofv3 --pmc " + " ".join(PMC_PASSES[0]) + " --kernel-include-regex "
                "'tile_|bwd_|wt_prep|dxc_|conv_bwd|dw_|colsum' -d OUT/bpmc1 -o run --output-format "
                "csv -- python3 REPO/bench.py --steps 2 --warmup 1 --no-cpu-baseline --settle-s 0 --no-decode "
                "--no-mqa --no-plan-legs --bwd-warmup 2 --bwd-reps 3",
    "bwd_pmc2": "rocprofv3 --pmc " + " ".join(PMC_PASSES[1]) + " --kernel-include-regex "
                "'tile_|bwd_|wt_prep|dxc_|conv_bwd|dw_|colsum' -d OUT/bpmc2 -o run --output-format "
                "csv -- python3 REPO/bench.py --steps 2 --warmup 1 --no-cpu-baseline --settle-s 0 --no-decode "
                "--no-mqa --no-plan-legs --bwd-warmup 2 --bwd-reps 3",
    "pmc1": "rocprofv3 --pmc " + " ".join(PMC_PASSES[0]) + " -d OUT/pmc1 -o run "
            "--output-format csv -- python3 REPO/bench.py --steps 5 --warmup 2 --no-cpu-baseline --settle-s 0 "
            "--no-backward --no-decode --no-mqa --no-plan-legs",
    "pmc2": "rocprofv3 --pmc " + " ".join(PMC_PASSES[1]) + " -d OUT/pmc2 -o run "
            "--output-format csv -- python3 REPO/bench.py --steps 5 --warmup 2 --no-cpu-baseline --settle-s 0 "
            "--no-backward --no-decode --no-mqa --no-plan-legs",
}


def _counter_rows(path):
    import csv
    return list(csv.DictReader(open(path)))


def traffic_summary(fetch_csv, write_csv, workload, copy_mib=256):
    """HBM bytes per launch of the fused kernel from two rocprofv3 counter passes (FETCH_SIZE and
    WRITE_SIZE, KiB per dispatch), each scaled by what the same counter reads for the device copy
    of copy_mib MiB in the same run (which reads and writes exactly copy_mib MiB)."""
    out = {}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = [r for r in _counter_rows(path) if r["Counter_Name"] == name]
        fused = [float(r["Counter_Value"]) for r in rows
                 if is_fused_kernel(r["Kernel_Name"]) and "fused_reset" not in r["Kernel_Name"]]
        copy = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        if not fused or not copy:
            raise SystemExit(f"{path}: no fused_forward or copy dispatches with {name}")
        copy_kib = max(copy)  # the calibration copies are by far the largest
        factor = copy_mib * 1024.0 / copy_kib
        out[name] = (sum(fused) / len(fused), len(fused), copy_kib, factor)
    hbm = sum(v[0] * v[3] for v in out.values()) * 1024.0
    path = os.path.join(ROOT, "profiles", f"traffic_fused_{workload}.txt")
    with open(path, "w") as f:
        f.write("# HBM traffic of the fused forward kernel, from rocprofv3 counters.\n")
        f.write("# Made by (REPO = this repository, OUT = a scratch directory; run from /tmp):\n")
        f.write(f"#   {PROFILE_CMDS['fetch']}\n#   {PROFILE_CMDS['write']}\n")
        f.write("#   python3 REPO/bench.py --traffic-summary OUT/fetch/fetch_counter_collection.csv "
                "OUT/write/write_counter_collection.csv\n")
        f.write("# Each counter (KiB per dispatch, summed over the chip) is scaled by copy MiB * 1024 /\n"
                "# what it reads for the device copy of that size in the same run.\n")
        f.write(f"workload: {workload}\n")
        f.write(f"source_hash: {kernel_source_hash()}\n")
        for name, (kib, n, copy_kib, factor) in out.items():
            f.write(f"{name.lower()}_kib_per_launch: {kib:.1f}\n")
            f.write(f"{name.lower()}_dispatches: {n}\n")
            f.write(f"{name.lower()}_copy_{copy_mib}mib_kib: {copy_kib:.1f}\n")
            f.write(f"{name.lower()}_calibration_factor: {factor:.4f}\n")
        f.write(f"hbm_bytes_per_launch: {hbm:.0f}\n")
    print(open(path).read(), end="")


def backward_traffic_summary(fetch_csv, write_csv, workload, copy_mib=256):
    """HBM bytes of one rglru_backward call: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) summed
    over the backward's kernels, per call (dispatches of each kernel / calls), each counter scaled
    by what it reads for the device copy of copy_mib MiB in the same run."""
    import collections
    per_kernel = collections.defaultdict(dict)
    factors = {}
    calls = None
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = [r for r in _counter_rows(path) if r["Counter_Name"] == name]
        copy = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        if not copy:
            raise SystemExit(f"{path}: no copy dispatches with {name}")
        factors[name] = copy_mib * 1024.0 / max(copy)
        sums, counts = collections.defaultdict(float), collections.Counter()
        for r in rows:
            if is_backward_kernel(r["Kernel_Name"]):
                k = r["Kernel_Name"].replace("void ", "").split("(")[0]
                sums[k] += float(r["Counter_Value"])
                counts[k] += 1
        calls = max(counts.values()) if counts else 0
        for k in sums:
            per_kernel[k][name] = sums[k] / calls * factors[name] * 1024.0  # bytes per call
    total = sum(v.get("FETCH_SIZE", 0.0) + v.get("WRITE_SIZE", 0.0) for v in per_kernel.values())
    path = os.path.join(ROOT, "profiles", f"traffic_backward_{workload}.txt")
    with open(path, "w") as f:
        f.write("# HBM traffic of one rglru_backward call, from rocprofv3 counters.\n")
        f.write("# Made by (REPO = this repository, OUT = a scratch directory; run from /tmp):\n")
        f.write(f"#   {PROFILE_CMDS['bwd_fetch']}\n#   {PROFILE_CMDS['bwd_write']}\n")
        f.write("#   python3 REPO/bench.py --backward-traffic-summary "
                "OUT/bfetch/fetch_counter_collection.csv OUT/bwrite/write_counter_collection.csv\n")
        f.write("# Counters are KiB per dispatch summed over the chip, scaled by copy MiB * 1024 / the\n"
                "# counter's reading for the device copy of that size in the same run.\n")
        f.write(f"workload: {workload}\n")
        f.write(f"source_hash: {kernel_source_hash(BACKWARD_SOURCES)}\n")
        f.write(f"calls: {calls}\n")
        for name, fac in factors.items():
            f.write(f"{name.lower()}_calibration_factor: {fac:.4f}\n")
        f.write(f"{'read_MB':>9} {'write_MB':>9}  kernel\n")
        for k, v in sorted(per_kernel.items(), key=lambda kv: -sum(kv[1].values())):
            f.write(f"{v.get('FETCH_SIZE', 0) / 1e6:9.1f} {v.get('WRITE_SIZE', 0) / 1e6:9.1f}  {k}\n")
        f.write(f"hbm_bytes_per_call: {total:.0f}\n")
    print(open(path).read(), end="")


def counter_summary(p1_csv, p2_csv, workload, backward=False):
    """Per-launch instruction and busy counts of every kernel of the bench's forward (fused plan
    and the split plan's stages) -- or, with backward, of one rglru_backward call -- from the two
    counter passes of PMC_PASSES, with the derived rates. The first dispatch of each kernel (cold
    caches, code load) is left out."""
    import collections
    from workloads import WORKLOADS
    w = [v for v in WORKLOADS.values() if v.name == workload][0]
    n = w.B * w.T * w.D
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    dur = collections.defaultdict(list)
    for p, path in ((1, p1_csv), (2, p2_csv)):
        disp = collections.defaultdict(dict)
        for r in _counter_rows(path):
            if "rglru::" not in r["Kernel_Name"]:
                continue  # torch's input set-up, the runtime's copies
            if backward != is_backward_kernel(r["Kernel_Name"]):
                continue
            k = r["Kernel_Name"].replace("void ", "").split("(")[0].replace("rglru::", "")
            disp[(k, r["Dispatch_Id"])][r["Counter_Name"]] = float(r["Counter_Value"])
            disp[(k, r["Dispatch_Id"])]["_ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        seen = set()
        for (k, did) in sorted(disp, key=lambda kd: int(kd[1])):
            if k not in seen:
                seen.add(k)
                continue
            for c, v in disp[(k, did)].items():
                if c == "_ns":
                    if p == 1:
                        dur[k].append(v)
                else:
                    vals[k][f"p{p}:{c}"].append(v)
    mean = lambda xs: sum(xs) / len(xs) if xs else float("nan")
    tag = "backward_" if backward else ""
    cmds = ("bwd_pmc1", "bwd_pmc2") if backward else ("pmc1", "pmc2")
    path = os.path.join(ROOT, "profiles", f"counters_{tag}{workload}.txt")
    with open(path, "w") as f:
        f.write("# Instruction and busy counters per launch of the "
                f"{'backward' if backward else 'forward'}'s kernels (rocprofv3).\n")
        f.write("# Made by (REPO = this repository, OUT = a scratch directory; run from /tmp):\n")
        f.write(f"#   {PROFILE_CMDS[cmds[0]]}\n#   {PROFILE_CMDS[cmds[1]]}\n")
        f.write(f"#   python3 REPO/bench.py --{'backward-' if backward else ''}counter-summary "
                f"OUT/{'b' if backward else ''}pmc1/run_counter_collection.csv "
                f"OUT/{'b' if backward else ''}pmc2/run_counter_collection.csv\n")
        f.write("# Means over the dispatches of each kernel after its first. Derived rates:\n"
                "#   cycles = GRBM_GUI_ACTIVE / 8 (one count per XCD); simd_cycles = 1024 * cycles\n"
                "#   mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / simd_cycles\n"
                f"#   valu_issue = ({VALU_CYCLES:g} * (VALU - MFMA - TRANS) + {TRANS_CYCLES:g} * TRANS)"
                " / simd_cycles  (the issue model of the ALU roofline)\n"
                "#   valu_active_per_wave = SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES (share of a wave's\n"
                "#     life spent issuing VALU; both in quad-cycles)\n"
                "#   wait_any / wait_inst = SQ_WAIT_ANY / SQ_WAIT_INST_ANY over SQ_WAVE_CYCLES\n"
                "#   lds_bank_conflict = SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS\n"
                "#   per_element: over B*T*D of the workload\n")
        f.write(f"workload: {workload}\n")
        f.write(f"source_hash: {kernel_source_hash(BACKWARD_SOURCES if backward else None)}\n")
        for k in sorted(vals, key=lambda k: -mean(dur[k])):
            v = {c: mean(xs) for c, xs in vals[k].items()}
            valu, mfma = v.get("p1:SQ_INSTS_VALU", 0.0), v.get("p1:SQ_INSTS_MFMA", 0.0)
            trans = v.get("p2:SQ_INSTS_VALU_TRANS_F32", 0.0)
            cyc = v.get("p1:GRBM_GUI_ACTIVE", float("nan")) / XCDS
            simd_cyc = SIMDS * cyc
            issue = VALU_CYCLES * (valu - mfma - trans) + TRANS_CYCLES * trans
            wc1, wc2 = v.get("p1:SQ_WAVE_CYCLES", float("nan")), v.get("p2:SQ_WAVE_CYCLES",
                                                                         float("nan"))
            lds_act = v.get("p2:SQ_ACTIVE_INST_LDS", 0.0)
            f.write(f"[{k}]\n")
            f.write(f"  dispatches: {len(dur[k])}\n")
            f.write(f"  duration_us: {mean(dur[k]) / 1e3:.2f}\n")
            f.write(f"  clock_ghz_est: {cyc / mean(dur[k]):.3f}\n")
            f.write(f"  waves: {v.get('p1:SQ_WAVES', 0):.0f}\n")
            f.write(f"  valu_insts: {valu - mfma:.0f}\n")
            f.write(f"  trans_insts: {trans:.0f}\n")
            f.write(f"  mfma_insts: {mfma:.0f}\n")
            f.write(f"  salu_insts: {v.get('p1:SQ_INSTS_SALU', 0):.0f}\n")
            f.write(f"  lds_insts: {v.get('p1:SQ_INSTS_LDS', 0):.0f}\n")
            f.write(f"  valu_per_element: {(valu - mfma) * 64 / n:.2f}\n")
            f.write(f"  trans_per_element: {trans * 64 / n:.2f}\n")
            f.write(f"  mfma_busy: {v.get('p1:SQ_VALU_MFMA_BUSY_CYCLES', 0) / simd_cyc:.4f}\n")
            f.write(f"  valu_issue: {issue / simd_cyc:.4f}\n")
            f.write(f"  valu_active_per_wave: {v.get('p1:SQ_ACTIVE_INST_VALU', 0) / wc1:.4f}\n")
            f.write(f"  wait_any: {v.get('p2:SQ_WAIT_ANY', 0) / wc2:.4f}\n")
            f.write(f"  wait_inst: {v.get('p2:SQ_WAIT_INST_ANY', 0) / wc2:.4f}\n")
            f.write(f"  lds_bank_conflict: "
                    f"{(v.get('p2:SQ_LDS_BANK_CONFLICT', 0) / lds_act) if lds_act else 0.0:.4f}\n")
    print(open(path).read(), end="")


def measured_counters(kernel: str, workload: str):
    """The [kernel] block of the committed counter summary as a dict of floats, if it was taken on
    the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"counters_{workload}.txt")
    if not os.path.exists(path):
        return None
    out, cur, top = {}, None, {}
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        if line.startswith("["):
            cur = line.strip()[1:-1]
            out[cur] = {}
        elif ":" in line:
            k, v = (t.strip() for t in line.split(":", 1))
            (out[cur] if cur else top)[k] = v
    if top.get("source_hash") != kernel_source_hash():
        return None
    blk = next((b for name, b in out.items() if name.startswith(kernel)), None)
    try:
        return {k: float(v) for k, v in blk.items()} if blk else None
    except ValueError:
        return None


def trace_summary(stats_csv, workload, bench_line_path=None, key="rg2b"):
    """Condensed rocprofv3 --kernel-trace --stats summary (per-kernel calls and durations)."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    path = os.path.join(ROOT, "profiles", f"kernel_trace_fused_{workload}.txt")
    with open(path, "w") as f:
        f.write("# rocprofv3 kernel-trace statistics of the default bench run.\n")
        f.write("# Made by (REPO = this repository, OUT = a scratch directory; run from /tmp):\n")
        if key == "rg2b":
            f.write(f"#   {PROFILE_CMDS['trace']}\n")
            f.write("#   python3 REPO/bench.py --trace-summary OUT/trace/bench_kernel_stats.csv "
                    "[OUT/trace/stdout.txt]\n")
        else:
            f.write(f"#   {PROFILE_CMDS['leg_trace'].replace('_W', '_' + key).replace(' W ', ' ' + key + ' ')}\n")
            f.write(f"#   python3 REPO/bench.py --workload {key} --trace-summary "
                    f"OUT/trace_{key}/bench_kernel_stats.csv [OUT/trace_{key}/stdout.txt]\n")
        f.write(f"workload: {workload}\n")
        f.write(f"source_hash: {kernel_source_hash()}\n")
        f.write("# the library's kernels only (the bench's own torch kernels and its clock-settle\n"
                "# matrix product and copies are left out)\n")
        f.write(f"{'calls':>7} {'avg_us':>9} {'min_us':>9} {'max_us':>9}  kernel\n")
        for r in rows:
            if "rglru::" not in r["Name"]:
                continue
            name = r["Name"].split("(")[0].replace("void ", "")
            f.write(f"{int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:9.2f} "
                    f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f}  {name}\n")
        per_call = sum(float(r["AverageNs"]) for r in rows if is_fused_kernel(r["Name"])) / 1e3
        f.write(f"fused_call_us (fused_forward + fused_reset, one rglru_forward): {per_call:.2f}\n")
        bwd = sum(float(r["AverageNs"]) for r in rows if is_backward_kernel(r["Name"])) / 1e3
        f.write(f"backward_call_us (sum of the averages of the backward's kernels, one "
                f"rglru_backward): {bwd:.2f}\n")
        if bench_line_path:
            for line in open(bench_line_path):
                if line.startswith('{"metric"'):
                    d = json.loads(line)
                    f.write(f"bench_ms_per_step: {d['ms_per_step']}\n")
                    f.write(f"bench_roofline_kernel_ms: {d['roofline']['kernel_ms']}\n")
                    if "backward" in d:
                        f.write(f"bench_backward_ms: {d['backward']['ms']}\n")
    print(open(path).read(), end="")


def settle_clocks(torch, dev, seconds):
    """Keep the GPU busy for `seconds` of wall time with work that is not the measured path (a
    bf16 matrix product and a 256 MiB device copy, alternating), so that its clocks have left
    idle before the warm-up steps; the driver's short warm-ups (a handful of ~0.1 ms steps) end
    while the clocks are still ramping. Returns the seconds spent."""
    if seconds <= 0:
        return 0.0
    a = torch.randn(4096, 4096, device=dev).to(torch.bfloat16)
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            torch.matmul(a, a)
            dst.copy_(src)
        torch.cuda.synchronize()
    del a, src, dst
    return time.perf_counter() - t0


def decode_leg(torch, rg, reps=3):
    """The batched decode step on its workload (1024 rows, D=4096, 16 heads, 256 consecutive
    in-place steps): every step of the workload is timed, after one untimed pass."""
    from workloads import WORKLOADS, make_inputs, to_device
    w = WORKLOADS["decode"]
    g = to_device(make_inputs(w, seed=0), torch.device("cuda:0"))
    cs, h = g["conv_state"].clone(), g["h0"].clone()
    y_t = torch.empty_like(g["x"][0])

    def step(t):
        rg.rglru_decode_step(g["x"][t], cs, h, y_t, g["conv_w"], g["W_a"], g["b_a"], g["W_x"],
                             g["b_x"], g["Lam"])

    for t in range(w.T):
        step(t)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        for t in range(w.T):
            step(t)
    ev1.record()
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / (reps * w.T)
    Dh = w.D // w.H
    # per row and channel: x_t 2 B, conv_state 3 rows in and out 12 B, h in and out 8 B, y_t 2 B;
    # per step: the gate weights 2 H Dh^2 bf16
    nbytes = w.B * w.D * 24 + 2 * w.H * Dh * Dh * 2
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": w.name, "us_per_step": round(us, 2),
            "rows_per_s": round(w.B / (us * 1e-6), 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes": nbytes}}


def backward_leg(torch, rg, w, g, y, warmup=200, reps=100):
    """rglru_backward on the same workload, from the forward's y and seeded dy, dh_T: the whole
    call (all its kernels) timed with events on the current stream. Algorithmic bytes: x, y and
    dy in and dx out (I/O dtype), the parameters in, their fp32 gradients out, dh_T in, dh0
    out."""
    B, T, D, H = w.B, w.T, w.D, w.H
    Dh = D // H
    io = g["x"].dtype
    gen = torch.Generator(device="cuda").manual_seed(1)
    dy = torch.randn(g["x"].shape, generator=gen, device="cuda", dtype=torch.float32).to(io)
    dh_T = torch.randn((B, D), generator=gen, device="cuda", dtype=torch.float32)
    ws = torch.empty(rg.rglru_backward_workspace_size(B, T, D, H, io), dtype=torch.uint8,
                     device="cuda")

    def call():
        return rg.backward(g["x"], g["conv_w"], g["W_a"], g["b_a"], g["W_x"], g["b_x"], g["Lam"],
                           g["h0"], y, dy, dh_T, workspace=ws)

    out = call()
    for _ in range(warmup):
        rg.rglru_backward(g["x"], g["conv_w"], g["W_a"], g["b_a"], g["W_x"], g["b_x"], g["Lam"],
                          g["h0"], y, dy, dh_T, out["dx"], out["dconv_w"], out["dW_a"],
                          out["db_a"], out["dW_x"], out["db_x"], out["dLam"], out["dh0"], ws)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        rg.rglru_backward(g["x"], g["conv_w"], g["W_a"], g["b_a"], g["W_x"], g["b_x"], g["Lam"],
                          g["h0"], y, dy, dh_T, out["dx"], out["dconv_w"], out["dW_a"],
                          out["db_a"], out["dW_x"], out["db_x"], out["dLam"], out["dh0"], ws)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / reps
    n = B * T * D
    eb = 2 if io == torch.bfloat16 else 4
    params = 2 * H * Dh * Dh * eb + 4 * D * eb + 3 * 4 * D
    grads = 2 * H * Dh * Dh * 4 + 4 * D * 4 + 3 * 4 * D
    nbytes = 4 * n * eb + params + grads + 2 * 4 * B * D
    gbs = nbytes / (ms * 1e-3) / 1e9
    traffic = measured_traffic("backward", w.name, "hbm_bytes_per_call", BACKWARD_SOURCES)
    # The three gate contractions of the backward, 2 n 2Dh flops each: the pre-activations
    # recomputed, dxc = dp W, dW = dp^T xc. Executed on the matrix cores (bf16 I/O, Dh in {128,
    # 256}): the pre-activations twice (conv output as bf16 hi + lo) and dxc one half again (each
    # tile also computes three rows of the next one), 4.5 contractions in all.
    flops = 3 * 2.0 * n * 2 * Dh
    executed = 4.5 * 2.0 * n * 2 * Dh if io == torch.bfloat16 and Dh in (128, 256) else None
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": w.name, "ms": round(ms, 4), "value": n / (ms * 1e-3),
            "unit": "tokens·channels/s", "reps": reps, "warmup": warmup,
            "workspace_bytes": ws.numel(),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes": nbytes, "traffic": traffic,
                         "note": "whole backward call (all kernels) against x, y, dy in + dx out; "
                                 "traffic = measured HBM bytes of all its kernels per call"},
            "roofline_mfma": {"bound": "mfma", "achieved": round(tf, 1),
                              "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                              "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                              "algorithmic_flops": flops, "executed_flops": executed,
                              "executed_frac": (round(executed / (ms * 1e-3) / 1e12
                                                      / MFMA_BF16_PEAK_TFLOPS, 4)
                                                if executed else None)}}


def mqa_leg(torch, rg, warmup=20, reps=50):
    """Local sliding-window multi-query attention (rglru_local_mqa) on the Griffin-2B-shaped
    attention layer: B=8, T=2048, 10 query heads of 256 sharing one key/value head, window 1024,
    bf16, seeded N(0,1) inputs. Roofline: MFMA (bf16 dense peak) against the algorithmic flops
    4 * B * Hq * dh * (number of visible (query, key) pairs); the kernel issues up to 1.5x that
    in MFMA work (the probabilities enter the second contraction as bf16 hi + lo in the query
    blocks whose rows see fewer than 256 keys, 2 of the 16 here)."""
    from workloads import make_attention_inputs
    B, T, Hq, dh, W = 8, 2048, 10, 256, 1024
    inp = make_attention_inputs(B, T, Hq, dh, seed=0)
    q = torch.from_numpy(inp["q"]).to("cuda", torch.bfloat16)
    k = torch.from_numpy(inp["k"]).to("cuda", torch.bfloat16)
    v = torch.from_numpy(inp["v"]).to("cuda", torch.bfloat16)
    o = torch.empty_like(q)
    for _ in range(warmup):
        rg.rglru_local_mqa(q, k, v, o, W)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        rg.rglru_local_mqa(q, k, v, o, W)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / reps
    pairs = sum(min(t + 1, W) for t in range(T))
    flops = 4.0 * B * Hq * dh * pairs
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": f"local_mqa_b{B}_t{T}_hq{Hq}_dh{dh}_w{W}_bf16", "ms": round(ms, 4),
            "value": B * T * Hq / (ms * 1e-3), "unit": "query rows/s", "reps": reps,
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                         "algorithmic_flops": flops}}


def plan_legs(torch, rg, names=("long", "rg9b"), warmup=10, reps=30):
    """The long-sequence (B1 T65536) and 9B-shaped (B16 T4096 D4096) layers under the fused plan
    and the chunked split plan, each call bracketed by events on the launch stream, with its HBM
    roofline on the plan's algorithmic bytes, and the plan the automatic choice takes."""
    from workloads import WORKLOADS, make_inputs, to_device
    out = {}
    for name in names:
        w = WORKLOADS[name]
        inp = make_inputs(w, seed=0)
        g = to_device(inp)
        del inp
        B, T, D, H = w.B, w.T, w.D, w.H
        io = g["x"].dtype
        n = B * T * D
        eb, pb = (2, 4) if io == torch.bfloat16 else (4, 8)
        param_bytes = 2 * H * (D // H) ** 2 * eb + 4 * D * eb + 3 * 4 * D
        state_bytes = (8 if g["h0"] is not None else 4) * B * D
        y = torch.empty_like(g["x"])
        hT = torch.empty((B, D), dtype=torch.float32, device=g["x"].device)
        auto, _ = rg.rglru_forward_plan_info(B, T, D, H, io)
        leg = {"workload": w.name, "auto_plan": auto}
        for plan in ("fused", "chunked"):
            nb = rg.rglru_forward_workspace_size_planned(B, T, D, H, io, plan, 0)
            if nb == 0:
                leg[plan] = None
                continue
            ws = torch.empty(nb, dtype=torch.uint8, device=g["x"].device)

            def call():
                rg.rglru_forward_planned(g["x"], g["conv_w"], g["W_a"], g["b_a"], g["W_x"],
                                         g["b_x"], g["Lam"], g["h0"], y, hT, ws, plan, 0)

            for _ in range(warmup):
                call()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                call()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            if plan == "fused":  # x in, y out, once
                nbytes = n * 2 * eb + param_bytes + state_bytes
            else:  # gates: x in, pre-activations out; scan: x and pre-activations in, y out
                nbytes = n * (3 * eb + 2 * pb) + 2 * param_bytes + state_bytes
            gbs = nbytes / (ms * 1e-3) / 1e9
            leg[plan] = {"ms": round(ms, 4), "algorithmic_bytes": nbytes, "gbs": round(gbs, 1),
                         "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                         "value": round(n / (ms * 1e-3), 1)}
            del ws
        timed = {p: leg[p]["ms"] for p in ("fused", "chunked") if leg.get(p)}
        leg["fastest"] = min(timed, key=timed.get) if timed else None
        out[name] = leg
        del g, y, hT
        torch.cuda.empty_cache()
    return out


def cpu_baseline(w, inp, min_seconds=10.0, one_thread_seconds=5.0):
    """The fp64 oracle, as it stands, on the host cores (OpenMP over (sequence, head)): whole
    forwards of the full workload, repeated until min_seconds of wall time have passed, reported
    as the mean rate; beside it the same oracle on one thread over a bounded sample (whole
    forwards of the workload's first sequence alone), and the 1-thread rate of the CPU-checkable
    fp32 configuration."""
    import oracle
    from workloads import WORKLOADS, make_inputs

    def rate(x, conv_w, W_a, b_a, W_x, b_x, Lam, h0, elements, seconds):
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.forward(x, conv_w, W_a, b_a, W_x, b_x, Lam, h0)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= seconds:
                return reps, dt, reps * elements / dt

    args = (inp["x"], inp["conv_w"], inp["W_a"], inp["b_a"], inp["W_x"], inp["b_x"], inp["Lam"],
            inp["h0"])
    cores = oracle.threads()
    reps, dt, v = rate(*args, w.elements, min_seconds)
    out = {"value": v, "unit": "tokens·channels/s", "cores": cores, "kind": "oracle",
           "seconds": round(dt, 3),
           "sample": f"{reps} full forwards of B={w.B} T={w.T} D={w.D} H={w.H}, fp64"}
    try:
        oracle.set_threads(1)
        one = tuple(a[:1] if (a is not None and k in (0, 7)) else a for k, a in enumerate(args))
        r1, d1, v1 = rate(*one, w.elements // w.B, one_thread_seconds)
        t = make_inputs(WORKLOADS["tiny"], seed=0)
        tt = WORKLOADS["tiny"]
        r2, d2, v2 = rate(t["x"], t["conv_w"], t["W_a"], t["b_a"], t["W_x"], t["b_x"], t["Lam"],
                          t["h0"], tt.elements, 1.0)
        out["one_thread"] = {"value": v1, "unit": "tokens·channels/s", "cores": 1,
                             "seconds": round(d1, 3),
                             "sample": f"{r1} forwards of one sequence (B=1) of the same workload"}
        out["one_thread_tiny"] = {"value": v2, "unit": "tokens·channels/s", "cores": 1,
                                  "seconds": round(d2, 3),
                                  "sample": f"{r2} forwards of {tt.name}"}
    finally:
        oracle.set_threads(cores)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    # the warm-up also brings the GPU clocks up to their steady state (a few hundred ms)
    ap.add_argument("--warmup", type=int, default=3000)
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="seconds of unrelated GPU work (matmul + copy) before the warm-up steps, "
                         "so that the clocks have left idle")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-step leg")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward leg")
    ap.add_argument("--no-mqa", action="store_true", help="skip the local-attention leg")
    ap.add_argument("--no-plan-legs", action="store_true",
                    help="skip the long-sequence and 9B-shaped layers under the fused and chunked "
                         "plans")
    ap.add_argument("--bwd-warmup", type=int, default=200)
    ap.add_argument("--bwd-reps", type=int, default=100)
    ap.add_argument("--backward-traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_backward_<workload>.txt from two counter CSVs")
    ap.add_argument("--workload", default="rg2b")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the timed region, copy a MIB-MiB device buffer three times (the "
                         "known-size reference for rocprofv3 byte counters)")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_fused_<workload>.txt from two rocprofv3 counter "
                         "passes and exit (no GPU needed)")
    ap.add_argument("--counter-summary", nargs=2, metavar=("PMC1_CSV", "PMC2_CSV"),
                    help="write profiles/counters_<workload>.txt from the two counter passes and "
                         "exit (no GPU needed)")
    ap.add_argument("--backward-counter-summary", nargs=2, metavar=("PMC1_CSV", "PMC2_CSV"),
                    help="write profiles/counters_backward_<workload>.txt likewise")
    ap.add_argument("--trace-summary", nargs="+", metavar="CSV",
                    help="write profiles/kernel_trace_fused_<workload>.txt from a rocprofv3 "
                         "kernel_stats.csv (and optionally the bench stdout) and exit")
    args = ap.parse_args()
    if (args.traffic_summary or args.trace_summary or args.backward_traffic_summary
            or args.counter_summary or args.backward_counter_summary):
        from workloads import WORKLOADS
        wname = WORKLOADS[args.workload].name
        if args.counter_summary:
            counter_summary(*args.counter_summary, wname)
        if args.backward_counter_summary:
            counter_summary(*args.backward_counter_summary, wname, backward=True)
        if args.traffic_summary:
            traffic_summary(*args.traffic_summary, wname)
        if args.backward_traffic_summary:
            backward_traffic_summary(*args.backward_traffic_summary, wname)
        if args.trace_summary:
            trace_summary(args.trace_summary[0], wname,
                          args.trace_summary[1] if len(args.trace_summary) > 1 else None,
                          args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards over batch and heads without communication)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gated_linear_recurrence_conv1d_amd as rg
    from workloads import WORKLOADS, make_inputs, to_device

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = make_inputs(w, seed=0)
    g = to_device(inp, dev)
    B, T, D, H = w.B, w.T, w.D, w.H
    io = g["x"].dtype
    R = 3
    xs = [g["x"]] + [torch.randn_like(g["x"], dtype=torch.float32).to(io) for _ in range(R - 1)]
    ys = [torch.empty_like(g["x"]) for _ in range(R)]
    hTs = [torch.empty((B, D), dtype=torch.float32, device=dev) for _ in range(R)]
    ws_bytes = rg.rglru_forward_workspace_size(B, T, D, H, io)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    plan, chunk = rg.rglru_forward_plan_info(B, T, D, H, io)

    def fwd(i):
        k = i % R
        rg.rglru_forward(xs[k], g["conv_w"], g["W_a"], g["b_a"], g["W_x"], g["b_x"], g["Lam"],
                         g["h0"], ys[k], hTs[k], ws)

    settled = settle_clocks(torch, dev, args.settle_s)
    for i in range(args.warmup):
        fwd(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        fwd(i)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps

    n = B * T * D
    eb = 2 if io == torch.bfloat16 else 4
    pb = 4 if io == torch.bfloat16 else 8
    wbytes = 2 * H * (D // H) ** 2 * eb
    param_bytes = wbytes + 4 * D * eb + 3 * 4 * D  # W_a, W_x, conv_w, b_a, b_x, Lambda
    state_bytes = (8 if g["h0"] is not None else 4) * B * D  # h0 (if any) in, h_T out
    kernels = {}
    if plan == "fused":
        # one launch does the whole path: x in, y out, parameters, state
        kernels["fused"] = {"ms": ms, "bytes": n * 2 * eb + param_bytes + state_bytes,
                            "note": "events bracket the look-back reset and the fused kernel"}

    # The split plan's two stages, each bracketed by events (the same kernels rglru_forward runs
    # with the DIRECT / CHUNKED plans), for comparison.
    pre = rg.pre_buffer(g["x"])
    splan, schunk = ("chunked", 0) if plan == "fused" else (plan, chunk)
    sws = torch.empty(max(1, rg.rglru_scan_workspace_size(B, T, D, H, io)), dtype=torch.uint8,
                      device=dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]

    def staged(i, e=None):
        k = i % R
        if e is not None:
            e[0].record()
        rg.rglru_gate_preacts(xs[k], g["conv_w"], g["W_a"], g["b_a"], g["W_x"], g["b_x"], pre)
        if e is not None:
            e[1].record()
        rg.rglru_scan_preacts(xs[k], pre, g["conv_w"], g["Lam"], g["h0"], ys[k], hTs[k], H, sws,
                              splan, schunk)
        if e is not None:
            e[2].record()

    for i in range(args.warmup):
        staged(i)
    torch.cuda.synchronize()
    for i in range(args.steps):
        staged(i, evs[i])
    torch.cuda.synchronize()
    gate_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    scan_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    kernels["split_scan"] = {"ms": scan_ms, "bytes": n * (eb + pb + eb) + param_bytes + state_bytes,
                             "plan": splan}
    kernels["split_gates"] = {"ms": gate_ms, "bytes": n * (eb + pb) + param_bytes,
                              "tflops": 2.0 * n * 2 * (D // H) / (gate_ms * 1e-3) / 1e12}
    # the dominant kernel of the plan rglru_forward actually ran
    if plan == "fused":
        dom = "fused"
    else:
        dom = "split_scan" if scan_ms >= gate_ms else "split_gates"
    kd = kernels[dom]
    achieved = kd["bytes"] / (kd["ms"] * 1e-3) / 1e9
    traffic = measured_traffic(dom, w.name)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic, "kernel": dom, "kernel_ms": round(kd["ms"], 4),
                "algorithmic_bytes": kd["bytes"]}

    # The fused kernel against its other two ceilings: the gate contraction on the matrix cores
    # (algorithmic flops, 2 * n * 2Dh) and the vector ALU (issue cycles of the instructions the
    # kernel executes, counted once by rocprofv3 on the current sources; null if the committed
    # counter summary was taken on other sources).
    extra_roofs = {}
    if plan == "fused":
        flops = 2.0 * n * 2 * (D // H)
        tf = flops / (ms * 1e-3) / 1e12
        extra_roofs["roofline_mfma"] = {"bound": "mfma", "achieved": round(tf, 1),
                                        "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                        "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                                        "flops": flops, "kernel": "fused"}
        cnt = measured_counters("fused_forward", w.name)
        alu = None
        if cnt:
            issue = (VALU_CYCLES * (cnt["valu_insts"] - cnt["trans_insts"])
                     + TRANS_CYCLES * cnt["trans_insts"])
            ach = issue / (ms * 1e-3) / 1e9
            peak = SIMDS * CLOCK_GHZ
            alu = {"bound": "alu", "achieved": round(ach, 1), "peak": peak,
                   "unit": "G SIMD-cycles/s", "frac": round(ach / peak, 4),
                   "valu_per_element": cnt["valu_per_element"],
                   "trans_per_element": cnt["trans_per_element"], "kernel": "fused"}
        extra_roofs["roofline_alu"] = alu

    line = {
        "metric": METRIC,
        "value": n / (ms * 1e-3),
        "unit": "tokens·channels/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "clock_settle_s": round(settled, 3),
        "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if io == torch.bfloat16 else "f32",
        "data": "synthetic (seeded; N(0,1) inputs, 1/fan-in weights)",
        "config": {"workload": w.name, "B": B, "T": T, "D": D, "H": H, "plan": plan,
                   "chunk_len": chunk, "state": "f32", "io": str(io).replace("torch.", ""),
                   "rotating_buffers": R},
        "roofline": roofline,
        **extra_roofs,
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv)
                        for kk, vv in v.items()} for k, v in kernels.items()},
        "wall_s_timed": round(wall, 4),
        "alg_gbs_end_to_end": round((n * 2 * eb + wbytes) / (ms * 1e-3) / 1e9, 1),
    }
    if not args.no_backward:
        line["backward"] = backward_leg(torch, rg, w, g, ys[0], args.bwd_warmup, args.bwd_reps)
    if not args.no_decode:
        line["decode"] = decode_leg(torch, rg)
    if not args.no_mqa:
        line["local_mqa"] = mqa_leg(torch, rg)
    if not args.no_plan_legs:
        line["plans"] = plan_legs(torch, rg)
    if args.copy_calibration:
        src = torch.empty(args.copy_calibration << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
