"""Benchmark of the causal selective-SSM hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  prefill  Mamba-1 2.8B layer shape (batch 4, L=2048, d_inner=5120, d_state=16,
           conv width 4, fp16 I/O, fp32 state): causal conv1d + SiLU, then the
           selective scan with the silu(z) gate; final state and conv tail
           written to the cache slots;
  decode   one token for 245 concurrent requests gathered from a 512-slot cache
           (conv cache fp16 [512,5120,3], state cache fp32 [512,5120,16]): conv
           update, then the selective state update.
Inputs are resident in HBM before the timed region.  Several independent
buffer sets are rotated between steps so that no step re-reads what the
previous one left in the 256 MB Infinity Cache.

Prints one JSON line.  ``value`` is the whole step's algorithmic HBM traffic
(every input read once, every output written once) divided by the step time,
in GB/s.  Also reported: decode tokens/s at batch 245 (245 tokens per
conv-update + state-update pass), per-kernel GB/s, the dominant kernel's
roofline and the float64 oracle timed on this host's cores on a bounded
sample of the same workload.
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

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
# fp32 vector FMA rate without packed-FP32 forms: 256 CUs x 4 SIMDs x 16 lanes
# x 2 flop x 2.4 GHz (the published 157.3 TFLOP/s counts packed FP32)
VALU_PEAK_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix rate, published
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {"selective_scan": ["scan.hip", "ssm_device.hpp", "ssm_kernels.hpp"],
                  "state_update": ["ssu.hip", "ssm_device.hpp", "ssm_kernels.hpp"],
                  "decode_step": ["ssu.hip", "ssm_device.hpp", "ssm_kernels.hpp"],
                  "conv1d_prefill": ["conv1d.hip", "ssm_device.hpp", "ssm_kernels.hpp"],
                  "conv1d_decode": ["conv1d.hip", "ssm_device.hpp", "ssm_kernels.hpp"],
                  "conv1d_varlen": ["conv1d.hip", "ssm_device.hpp", "ssm_kernels.hpp"],
                  "selective_scan_varlen": ["scan.hip", "ssm_device.hpp", "ssm_kernels.hpp"],
                  "chunked_scan": ["ssd.hip", "ssm_kernels.hpp"],
                  "layer_decode": ["gemm.hip", "layer.hip", "conv1d.hip", "ssu.hip", "ssm_device.hpp",
                                   "ssm_kernels.hpp"]}
# rocprofv3 kernel names of each kernel in the benchmarked configuration
KERNEL_SYMBOLS = {"selective_scan": "scan_kernel", "decode_step": "ssu_ilv_kernel",
                  "conv1d_prefill": "conv_rows_kernel"}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="target duration of the CPU oracle sample")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device copy (for counter calibration)")
    p.add_argument("--ssu-sweep", action="store_true",
                   help="time the Mamba-2 state update over batch, groups and cache dtype "
                        "and print one JSON line per point")
    p.add_argument("--no-varlen", action="store_true",
                   help="skip the packed variable-length prefill measurement")
    p.add_argument("--no-layer", action="store_true",
                   help="skip the whole decode-layer measurement")
    p.add_argument("--no-chunked", action="store_true",
                   help="skip the chunked Mamba-2 prefill measurement")
    p.add_argument("--only", choices=["prefill", "decode", "varlen", "layer", "chunked"],
                   default=None,
                   help="run only one half of the step (for profiling)")
    p.add_argument("--unfused-decode", action="store_true",
                   help="decode with the separate conv-update and state-update calls instead "
                        "of the fused decode step")
    p.add_argument("--profile-script", metavar="OUTDIR",
                   help="print the rocprofv3 commands whose output --summarize-profile reads")
    p.add_argument("--summarize-profile", metavar="OUTDIR",
                   help="turn rocprofv3 CSV output under OUTDIR into profiles/ summaries")
    return p.parse_args()


SQ_COUNTERS = ("SQ_WAVES SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_WAVE_CYCLES SQ_BUSY_CYCLES "
               "SQ_WAIT_INST_ANY SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT")


def profile_commands(out):
    """The rocprofv3 runs behind the committed profiles: a kernel trace with
    stats, then one counter per pass (FETCH_SIZE, WRITE_SIZE) on the step and
    on a plain 1 GiB device copy (the calibration), and the SQ counters of the
    prefill half."""
    b = "python -u bench.py --no-cpu-baseline --no-varlen --no-layer --no-chunked"
    pmc = "timeout -s KILL 120 rocprofv3 --pmc {c} -f csv -d {o}/{n} -o run -- {cmd}"
    return [
        ("trace", f"timeout -s KILL 180 rocprofv3 --kernel-trace --stats -f csv -d {out}/trace "
                  f"-o run -- {b} --steps 20 --warmup 5"),
        ("fetch", pmc.format(c="FETCH_SIZE", o=out, n="fetch", cmd=f"{b} --steps 3 --warmup 1")),
        ("write", pmc.format(c="WRITE_SIZE", o=out, n="write", cmd=f"{b} --steps 3 --warmup 1")),
        ("copy_fetch", pmc.format(c="FETCH_SIZE", o=out, n="copy_fetch",
                                  cmd="python -u bench.py --copy-calibration")),
        ("copy_write", pmc.format(c="WRITE_SIZE", o=out, n="copy_write",
                                  cmd="python -u bench.py --copy-calibration")),
        ("sq", pmc.format(c=SQ_COUNTERS, o=out, n="sq",
                          cmd=f"{b} --steps 3 --warmup 1 --only prefill")),
        ("varlen_trace", f"timeout -s KILL 180 rocprofv3 --kernel-trace --stats -f csv -d "
                         f"{out}/varlen_trace -o run -- python -u bench.py --only varlen "
                         f"--steps 20 --warmup 5"),
        ("layer_trace", f"timeout -s KILL 180 rocprofv3 --kernel-trace --stats -f csv -d "
                        f"{out}/layer_trace -o run -- python -u bench.py --only layer "
                        f"--steps 20 --warmup 5"),
        ("chunked_trace", f"timeout -s KILL 180 rocprofv3 --kernel-trace --stats -f csv -d "
                          f"{out}/chunked_trace -o run -- python -u bench.py --only chunked "
                          f"--steps 20 --warmup 5"),
    ]


def _trace_table(stats, symbols):
    """Rows (symbol, calls, avg, min, max us) of a kernel_stats.csv, pooled
    over the instantiations whose name contains each symbol."""
    rows = []
    for sym, excl in symbols:
        rs = [r for r in stats if sym in r["Name"] and not (excl and excl in r["Name"])]
        calls = sum(int(r["Calls"]) for r in rs)
        if calls:
            tot = sum(float(r["TotalDurationNs"]) for r in rs)
            rows.append(f"| {sym} | {calls} | {tot / calls / 1e3:.1f} | "
                        f"{min(float(r['MinNs']) for r in rs) / 1e3:.1f} | "
                        f"{max(float(r['MaxNs']) for r in rs) / 1e3:.1f} |")
    return rows


def _json_field(log, key):
    with open(log) as f:
        for ln in f:
            if ln.startswith("{") and key in ln:
                return json.loads(ln)[key]
    return {}


def _read_counters(path):
    import collections
    import csv

    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    with open(path) as f:
        for r in csv.DictReader(f):
            agg[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return agg


def _match(agg, symbol):
    """Counters of the kernels whose name contains symbol, all instantiations
    pooled: {counter: mean per dispatch}."""
    vals = {}
    for name, d in agg.items():
        if symbol in name:
            for c, v in d.items():
                vals.setdefault(c, []).extend(v)
    return {c: sum(v) / len(v) for c, v in vals.items()}, sum(len(v) for v in vals.values())


def summarize_profile(out):
    """Write profiles/<kernel>_traffic.json and profiles/*.md from the CSVs of
    the runs listed by profile_commands()."""
    import csv
    import glob

    os.makedirs(PROFILES, exist_ok=True)
    cmds = dict(profile_commands(out))
    import workloads as W

    pb, db = W.algorithmic_bytes(W.prefill()), W.algorithmic_bytes(W.decode())
    dspec = W.decode()
    alg = {"conv1d_prefill": pb["conv"], "selective_scan": pb["scan"],
           "decode_step": db["conv"] + db["ssu"] - 2 * dspec.batch * dspec.channels * 2}
    copy_bytes = 1 << 30
    cf, _ = _match(_read_counters(glob.glob(f"{out}/copy_fetch/*counter_collection.csv")[0]),
                   "copyBuffer")
    cw, _ = _match(_read_counters(glob.glob(f"{out}/copy_write/*counter_collection.csv")[0]),
                   "copyBuffer")
    f_factor = copy_bytes / (cf["FETCH_SIZE"] * 1024)
    w_factor = copy_bytes / (cw["WRITE_SIZE"] * 1024)
    fetch = _read_counters(glob.glob(f"{out}/fetch/*counter_collection.csv")[0])
    write = _read_counters(glob.glob(f"{out}/write/*counter_collection.csv")[0])
    stats = list(csv.DictReader(open(glob.glob(f"{out}/trace/*kernel_stats.csv")[0])))
    # source hashes of the kernels as profiled: from the benchmark line the
    # traced run printed (not from the tree as it is now)
    profiled_sha = {}
    with open(f"{out}/trace.log") as f:
        for ln in f:
            if ln.startswith("{") and '"kernels"' in ln:
                profiled_sha = {k: v.get("kernel_source_sha")
                                for k, v in json.loads(ln)["kernels"].items()}

    lines = ["# Kernel trace and HBM traffic: Mamba-1 2.8B layer step", "",
             "Workload: prefill conv1d+scan, batch 4 x L 2048, d_inner 5120, d_state 16, f16 "
             "I/O, f32 state; one decode step (fused conv update + state update, "
             "`decode_step`), 245 requests from a 512-slot cache.", "",
             "Commands (run from the repository root on the MI355X):", ""]
    for n, c in profile_commands(out):
        lines.append(f"    {c}")
    lines += ["", f"Calibration: a plain 1 GiB device copy reads FETCH_SIZE = {cf['FETCH_SIZE']:.0f} "
              f"KiB and WRITE_SIZE = {cw['WRITE_SIZE']:.0f} KiB per dispatch, so HBM bytes = "
              f"FETCH_SIZE x 1024 x {f_factor:.3f} + WRITE_SIZE x 1024 x {w_factor:.3f}.", "",
              "| kernel | calls | avg us | min us | max us | algorithmic MB | counter read MB | "
              "counter write MB | traffic / algorithmic |", "|---|---|---|---|---|---|---|---|---|"]
    for k, sym in KERNEL_SYMBOLS.items():
        rows = [r for r in stats if sym in r["Name"]]
        calls = sum(int(r["Calls"]) for r in rows)
        tot = sum(float(r["TotalDurationNs"]) for r in rows)
        avg = tot / calls / 1e3 if calls else float("nan")
        mn = min(float(r["MinNs"]) for r in rows) / 1e3 if rows else float("nan")
        mx = max(float(r["MaxNs"]) for r in rows) / 1e3 if rows else float("nan")
        fr, _ = _match(fetch, sym)
        wr, _ = _match(write, sym)
        rb = fr.get("FETCH_SIZE", float("nan")) * 1024 * f_factor
        wb = wr.get("WRITE_SIZE", float("nan")) * 1024 * w_factor
        lines.append(f"| {k} | {calls} | {avg:.1f} | {mn:.1f} | {mx:.1f} | {alg[k] / 1e6:.1f} | "
                     f"{rb / 1e6:.1f} | {wb / 1e6:.1f} | {(rb + wb) / alg[k]:.3f} |")
        rec = {"kernel": k, "kernel_source_sha": profiled_sha.get(k),
               "fetch_kib_per_dispatch": fr.get("FETCH_SIZE"),
               "write_kib_per_dispatch": wr.get("WRITE_SIZE"),
               "fetch_factor": f_factor, "write_factor": w_factor,
               "hbm_bytes_per_launch": rb + wb, "algorithmic_bytes_per_launch": alg[k],
               "avg_launch_us_trace": avg, "commands": [cmds["fetch"], cmds["write"],
                                                       cmds["copy_fetch"], cmds["copy_write"]]}
        with open(os.path.join(PROFILES, f"{k}_traffic.json"), "w") as f:
            json.dump(rec, f, indent=1)
    sq = _read_counters(glob.glob(f"{out}/sq/*counter_collection.csv")[0])
    lines += ["", "SQ counters of the selective scan (mean per dispatch; command above, `sq`):", ""]
    v, _ = _match(sq, KERNEL_SYMBOLS["selective_scan"])
    for c in sorted(v):
        lines.append(f"- {c}: {v[c]:.0f}")
    if v.get("SQ_WAVES"):
        lines.append(f"- VALU instructions per wave: {v['SQ_INSTS_VALU'] / v['SQ_WAVES']:.0f}")
    with open(os.path.join(PROFILES, "mamba1_layer_step_kernels.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))

    # packed variable-length prefill: its own traced run
    vstats = list(csv.DictReader(open(glob.glob(f"{out}/varlen_trace/*kernel_stats.csv")[0])))
    vline = {}
    with open(f"{out}/varlen_trace.log") as f:
        for ln in f:
            if ln.startswith("{") and "varlen_prefill" in ln:
                vline = json.loads(ln)["varlen_prefill"]
    vl = ["# Kernel trace: packed variable-length prefill (Mamba-1 2.8B layer)", "",
          f"Workload: {vline.get('workload')}; lengths {vline.get('lengths')}.", "",
          "Command (run from the repository root on the MI355X):", "",
          f"    {cmds['varlen_trace']}", "",
          "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    # aligned packed rows of at most 255 sequences: the row kernel, which
    # also fixes the starts and writes the caches; other packed rows: the
    # tiled kernel and its cache pass
    for sym in ("conv_rows_kernel", "conv_varlen_kernel", "conv_varlen_tail_kernel", "scan_kernel"):
        rows = [r for r in vstats if sym in r["Name"] and
                (sym != "conv_varlen_kernel" or "tail" not in r["Name"])]
        calls = sum(int(r["Calls"]) for r in rows)
        tot = sum(float(r["TotalDurationNs"]) for r in rows)
        if calls:
            vl.append(f"| {sym} | {calls} | {tot / calls / 1e3:.1f} | "
                      f"{min(float(r['MinNs']) for r in rows) / 1e3:.1f} | "
                      f"{max(float(r['MaxNs']) for r in rows) / 1e3:.1f} |")
    if vline:
        vl += ["", f"Event-timed in the same run: conv1d (the whole call) "
                   f"{vline['conv1d_varlen']['us']:.1f} us for {vline['conv1d_varlen']['bytes'] / 1e6:.1f} MB, "
                   f"scan {vline['selective_scan_varlen']['us']:.1f} us for "
                   f"{vline['selective_scan_varlen']['bytes'] / 1e6:.1f} MB; "
                   f"{vline['tokens_per_s'] / 1e6:.1f} M tokens/s."]
    with open(os.path.join(PROFILES, "mamba1_varlen_prefill_kernels.md"), "w") as f:
        f.write("\n".join(vl) + "\n")
    print("\n".join(vl))

    # whole decode layer and chunked Mamba-2 prefill: their own traced runs
    for name, key, title, fname, syms in (
            ("layer_trace", "layer_decode", "whole Mamba-1 2.8B decode layer", "mamba1_decode_layer_kernels.md",
             [("rmsnorm_kernel", None), ("gemm_kernel", None), ("gemm_reduce_kernel", None),
              ("conv_decode", None), ("ssu_ilv_kernel", None)]),
            ("chunked_trace", "chunked_prefill", "chunked Mamba-2 prefill on MFMA",
             "mamba2_chunked_prefill_kernels.md", [("ssd_kernel", None)])):
        st = list(csv.DictReader(open(glob.glob(f"{out}/{name}/*kernel_stats.csv")[0])))
        rec = _json_field(f"{out}/{name}.log", key)
        ml = [f"# Kernel trace: {title}", "", f"Workload: {rec.get('workload')}.", "",
              "Command (run from the repository root on the MI355X):", "", f"    {cmds[name]}", "",
              "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
        ml += _trace_table(st, syms)
        # every library kernel in the run, by name (the rest set up inputs)
        ml += ["", "All library kernels of the run (name, calls, avg us):", ""]
        for r in sorted(st, key=lambda r: -float(r["TotalDurationNs"])):
            if "ssm" not in r["Name"]:
                continue
            ml.append(f"- `{r['Name'][:120]}`: {r['Calls']}, {float(r['AverageNs']) / 1e3:.1f}")
        if rec:
            ml += ["", f"Event-timed in the same run: {rec['us']:.1f} us per call"
                       + (f", {rec['tokens_per_s'] / 1e6:.2f} M tokens/s" if "tokens_per_s" in rec else "")
                       + (f", {rec['GBps']:.0f} GB/s of algorithmic traffic" if "GBps" in rec else "")
                       + (f", {rec['mfma_TFLOPs']:.0f} TFLOP/s of algorithmic MFMA work"
                          if "mfma_TFLOPs" in rec else "") + "."]
        with open(os.path.join(PROFILES, fname), "w") as f:
            f.write("\n".join(ml) + "\n")
        print("\n".join(ml))


def kernel_source_sha(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "state_space_model_causal_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, sha: str, launches_per_step: int = 1):
    """Counter-measured HBM bytes per launch, if the committed measurement was
    taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, f"{kernel}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.profile_script:
        for n, c in profile_commands(args.profile_script):
            print(f'echo "step: {n}" && {c} > {args.profile_script}/{n}.log 2>&1 || exit 1')
        return
    if args.summarize_profile:
        summarize_profile(args.summarize_profile)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    from state_space_model_causal_amd import LIB_PATH
    if not os.path.exists(LIB_PATH):
        from state_space_model_causal_amd import build as hip_build
        hip_build.build()
    import state_space_model_causal_amd as ssm
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 10
        print(json.dumps({"copy_bytes_each_way": n, "ms": ms, "GBps": 2 * n / ms / 1e6}), flush=True)
        return

    pspec = W.prefill()
    dspec = W.decode()
    pbytes = W.algorithmic_bytes(pspec)
    dbytes = W.algorithmic_bytes(dspec)

    stream = torch.cuda.current_stream()
    if args.ssu_sweep:
        ssu_sweep(ssm, W, dev, stream)
        return
    if args.only == "layer":
        print(json.dumps({"layer_decode": measure_layer(ssm, W, dev, stream, args.steps,
                                                        args.warmup)}), flush=True)
        return
    if args.only == "chunked":
        print(json.dumps({"chunked_prefill": measure_chunked(ssm, W, dev, stream, args.steps,
                                                             args.warmup)}), flush=True)
        return
    if args.only == "varlen":
        print(json.dumps({"varlen_prefill": measure_varlen(ssm, W, dev, stream, args.steps,
                                                           args.warmup)}), flush=True)
        return

    # buffer sets: 2 prefill sets (~0.5 GB each) and 3 decode sets (~0.19 GB)
    NP, ND = 2, 3
    psets, dsets = [], []
    for k in range(NP if args.only != "decode" else 0):
        t = W.make(W.prefill(seed=pspec.seed + 100 * k), dev)
        t["u"] = torch.empty_like(t["x"])
        t["out"] = torch.empty_like(t["x"])
        psets.append(t)
    for k in range(ND if args.only != "prefill" else 0):
        t = W.make(W.decode(seed=dspec.seed + 100 * k), dev)
        t["x3"] = t["x"].view(dspec.batch, dspec.channels, 1)
        t["u"] = torch.empty_like(t["x3"])
        t["out"] = torch.empty_like(t["x"])
        dsets.append(t)
    torch.cuda.synchronize()

    fused = not args.unfused_decode

    def step(i, ev=None):
        # ev: 5 events bracketing prefill conv, prefill scan, then either the
        # fused decode step (3 -> 4) or conv update (2 -> 3) + state update (3 -> 4)
        def rec(j):
            if ev is not None:
                ev[j].record(stream)
        rec(0)
        if psets:
            t = psets[i % NP]
            ssm.causal_conv1d(t["x"], t["conv_w"], t["conv_b"], conv_state=t["conv_state"],
                              slot_idx=t["slot_idx"], out=t["u"], has_initial_state=False,
                              stream=stream)
            rec(1)
            ssm.selective_scan(t["u"], t["dt"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                               dt_bias=t["dt_bias"], ssm_state=t["ssm_state"],
                               slot_idx=t["slot_idx"], has_initial_state=False, out=t["out"],
                               stream=stream)
        else:
            rec(1)
        rec(2)
        if dsets:
            t = dsets[i % ND]
            if fused:
                rec(3)
                ssm.decode_step(t["ssm_state"], t["conv_state"], t["x"], t["conv_w"], t["dt"],
                                t["A"], t["B"], t["C"], conv_bias=t["conv_b"], D=t["D"],
                                z=t["z"], dt_bias=t["dt_bias"], slot_idx=t["slot_idx"],
                                out=t["out"], stream=stream)
            else:
                ssm.causal_conv1d(t["x3"], t["conv_w"], t["conv_b"], conv_state=t["conv_state"],
                                  slot_idx=t["slot_idx"], out=t["u"], has_initial_state=True,
                                  stream=stream)
                rec(3)
                ssm.state_update(t["ssm_state"], t["u"].view(dspec.batch, dspec.nheads, 1),
                                 t["dt"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                 dt_bias=t["dt_bias"], slot_idx=t["slot_idx"], out=t["out"],
                                 stream=stream)
        else:
            rec(3)
        rec(4)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    K = args.steps
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(K)]
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    for i in range(K):
        step(i, events[i])
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0

    per = np.array([[events[i][j].elapsed_time(events[i][j + 1]) for j in range(4)]
                    for i in range(K)])  # ms, [K, 4]: conv, scan, conv update, state update
    step_ms = np.array([events[i][0].elapsed_time(events[i][4]) for i in range(K)])
    total_ms = events[0][0].elapsed_time(events[K - 1][4])
    ms_per_step = total_ms / K
    k_ms = per.mean(axis=0)

    # the fused decode step moves the conv cache and the state, not u
    fused_bytes = dbytes["conv"] + dbytes["ssu"] - 2 * dspec.batch * dspec.channels * 2
    step_bytes = ((pbytes["conv"] + pbytes["scan"]) if psets else 0) + \
                 (((fused_bytes if fused else dbytes["conv"] + dbytes["ssu"])) if dsets else 0)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    def gbps(b, ms):
        return b / (ms * 1e-3) / 1e9 if ms > 0 else None

    kernels = {
        "conv1d_prefill": {"bytes": pbytes.get("conv"), "us": k_ms[0] * 1e3},
        "selective_scan": {"bytes": pbytes.get("scan"), "us": k_ms[1] * 1e3},
    }
    if fused:
        kernels["decode_step"] = {"bytes": fused_bytes, "us": k_ms[3] * 1e3}
    else:
        kernels["conv1d_decode"] = {"bytes": dbytes.get("conv"), "us": k_ms[2] * 1e3}
        kernels["state_update"] = {"bytes": dbytes.get("ssu"), "us": k_ms[3] * 1e3}
    for k, v in kernels.items():
        v["kernel_source_sha"] = kernel_source_sha(KERNEL_SOURCES[k])
        v["GBps"] = gbps(v["bytes"], v["us"] * 1e-3) if v["bytes"] else None
        v["frac_hbm_peak"] = v["GBps"] / HBM_PEAK_GBPS if v["GBps"] else None

    decode_ms = k_ms[2] + k_ms[3]  # conv update + state update, or the fused step
    decode_tps = dspec.batch / (decode_ms * 1e-3) if dsets else None

    # dominant kernel: the one with the largest share of the step
    dom = max(kernels, key=lambda k: kernels[k]["us"])
    dk = kernels[dom]
    sha = kernel_source_sha(KERNEL_SOURCES[dom])
    traffic = load_traffic(dom, sha)
    if dom == "selective_scan":
        # The Mamba-1 scan is bound by float32 VALU work, not by HBM: one
        # exponential (half-rate on gfx950) and four other VALU operations per
        # (time, channel, state) element against 8 bytes of HBM traffic per
        # (time, channel).  Its roofline is the non-packed fp32 FMA rate.
        flops = W.algorithmic_flops(pspec)
        achieved = flops / (dk["us"] * 1e-6) / 1e12
        roofline = {"kernel": dom, "bound": "alu", "achieved": achieved,
                    "peak": VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": achieved / VALU_PEAK_TFLOPS, "traffic": traffic,
                    "algorithmic_flops_per_launch": flops,
                    "algorithmic_bytes_per_launch": dk["bytes"],
                    "hbm_GBps": dk["GBps"], "hbm_frac": dk["frac_hbm_peak"]}
    else:
        roofline = {"kernel": dom, "bound": "hbm", "achieved": dk["GBps"], "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": dk["frac_hbm_peak"], "traffic": traffic,
                    "algorithmic_bytes_per_launch": dk["bytes"]}
    roofline["avg_launch_us"] = dk["us"]
    roofline["kernel_source_sha"] = sha

    varlen = None
    if not args.no_varlen and args.only is None:
        varlen = measure_varlen(ssm, W, dev, stream, max(args.steps // 2, 5), 3)

    layer = None
    if not args.no_layer and args.only is None:
        layer = measure_layer(ssm, W, dev, stream, max(args.steps // 2, 5), 3)

    chunked = None
    if not args.no_chunked and args.only is None:
        chunked = measure_chunked(ssm, W, dev, stream, max(args.steps // 2, 5), 3)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.cpu_seconds, pspec, dspec)

    line = {
        "metric": "selective_scan/SSU HBM GB/s + % of roofline; decode tokens/s at batch 245",
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "io_dtype": "f16",
        "data": "synthetic (seeded; Mamba-2.8B layer shapes, random parameters)",
        "config": {
            "workload": "mamba1-2.8B layer: prefill conv1d+scan batch 4 x L 2048, d_inner 5120, "
                        "d_state 16, conv 4, f16 io / f32 state; + one decode step (conv update "
                        "+ state update), 245 requests from a 512-slot cache",
            "prefill": {"batch": pspec.batch, "seqlen": pspec.seqlen, "d_inner": pspec.channels,
                        "d_state": pspec.dstate, "conv_width": pspec.width},
            "decode": {"batch": dspec.batch, "nslots": dspec.nslots, "d_inner": dspec.channels,
                       "d_state": dspec.dstate, "fused_conv_update": fused},
            "step_bytes": step_bytes,
            "buffer_sets": {"prefill": NP, "decode": ND},
            "only": args.only,
        },
        "pct_hbm_roofline": value / HBM_PEAK_GBPS * 100,
        "decode_tokens_per_s": decode_tps,
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "varlen_prefill": varlen,
        "layer_decode": layer,
        "chunked_prefill": chunked,
        "step_ms_median": float(np.median(step_ms)),
        "wall_s_timed": t_wall,
        "device": props.name,
        "arch": getattr(props, "gcnArchName", None),
    }
    print(json.dumps(line), flush=True)


def ssu_sweep(ssm, W, dev, stream, iters=20):
    """Mamba-2 decode state update at the two head shapes (headdim 64 /
    dstate 128 with 80 heads; headdim 128 / dstate 256 with 64 heads) over
    batch, ngroups and cache dtype.  Each point rotates through disjoint slot
    sets covering at least 1 GB of cache, so no launch finds its state in the
    on-chip caches, and is timed as replays of a HIP graph of the launches."""
    import math

    import torch

    points = []
    shapes = [("hd64_N128", W.m2_ssu_64, (1, 8), ("f16", "f32"), (1, 16, 256, 1024)),
              ("hd128_N256", W.m2_ssu_128, (1,), ("bf16", "f32"), (1, 8, 64, 512))]
    for name, factory, groups, caches, batches in shapes:
        for G in groups:
            for cache in caches:
                for Bt in batches:
                    probe = factory(batch=Bt, state=cache, ngroups=G)
                    ssz = 4 if cache == "f32" else 2
                    per_req = 2 * probe.nheads * probe.headdim * probe.dstate * ssz
                    R = max(1, math.ceil(1e9 / (Bt * per_req)))
                    spec = factory(batch=Bt, state=cache, ngroups=G, nslots=Bt * R,
                                   random_slots=False)
                    t = W.make(spec, dev)
                    out = torch.empty_like(t["x"])
                    sets = [(torch.arange(Bt, dtype=torch.int32, device=dev) + r * Bt).contiguous()
                            for r in range(R)]

                    def run(i):
                        ssm.state_update(t["ssm_state"], t["x"], t["dt"], t["A"], t["B"], t["C"],
                                         D=t["D"], z=t["z"], dt_bias=t["dt_bias"],
                                         slot_idx=sets[i % R], out=out)

                    # a graph of `launches` launches, replayed: device time
                    # per launch, without the host's launch rate
                    for i in range(3):
                        run(i)
                    torch.cuda.synchronize()
                    launches = max(iters, R)
                    graph = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(graph):
                        for i in range(launches):
                            run(i)
                    graph.replay()
                    torch.cuda.synchronize()
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    for _ in range(3):
                        graph.replay()
                    e1.record()
                    torch.cuda.synchronize()
                    us = e0.elapsed_time(e1) * 1e3 / (3 * launches)
                    b = W.algorithmic_bytes(spec)["ssu"]
                    pt = {"shape": name, "ngroups": G, "cache": cache, "batch": Bt,
                          "effective_batch": Bt * spec.nheads, "us": us, "bytes": b,
                          "GBps": b / (us * 1e-6) / 1e9,
                          "pct_hbm": b / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS * 100,
                          "rotation_sets": R}
                    print(json.dumps({"ssu_sweep": pt}), flush=True)
                    points.append(pt)
                    del t, out, sets, graph
                    torch.cuda.empty_cache()
    return points


def measure_layer(ssm, W, dev, stream, steps, warmup):
    """One whole Mamba-1 2.8B decode layer (RMSNorm, in_proj, conv update,
    x_proj, dt_proj, state update, out_proj + residual; random weights) for
    245 requests from a 512-slot cache, f16 I/O and f32 state; two rotating
    sets of caches.  Timed with events on the launch stream."""
    import numpy as np
    import torch

    sets = [W.mamba1_layer(seed=30 + k, device=dev) for k in range(2)]
    descs = [ssm.mamba1_layer(t["w"]) for t in sets]
    lib = ssm.load_library()
    import ctypes
    need = lib.ssm_mamba1_decode_layer_workspace(ctypes.byref(descs[0]), 245)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)

    def run(i):
        t = sets[i % 2]
        ssm.mamba1_decode_layer(descs[i % 2], t["hidden"], t["conv_state"], t["ssm_state"],
                                slot_idx=t["slot_idx"], workspace=ws, stream=stream)

    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        run(i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    us = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]) * 1e3
    b = W.layer_bytes(2560, 5120, 16, 160, 4, 245)
    mean = float(us.mean())
    return {"workload": "Mamba-1 2.8B decode layer (d_model 2560, d_inner 5120, d_state 16, "
                        "dt_rank 160, conv 4), 245 requests, f16 I/O and weights, f32 state, "
                        "random weights",
            "us": mean, "us_median": float(np.median(us)), "tokens_per_s": 245 / (mean * 1e-6),
            "bytes": b["total"], "GBps": b["total"] / (mean * 1e-6) / 1e9,
            "model_tokens_per_s_64_layers": 245 / (64 * mean * 1e-6), "steps": steps}


def measure_chunked(ssm, W, dev, stream, steps, warmup):
    """Mamba-2 prefill in the chunked matrix form (the library's choice for
    bf16 I/O): 2 requests x L 4096, 64 heads of headdim 128, dstate 256,
    bf16 I/O, f32 state written to a 1024-slot cache; two rotating buffer
    sets, timed with events on the launch stream."""
    import numpy as np
    import torch

    spec = W.m2_prefill(state="f32")
    sets = []
    for k in range(2):
        t = W.make(W.m2_prefill(state="f32", seed=spec.seed + 100 * k), dev)
        t["out"] = torch.empty_like(t["x"])
        sets.append(t)

    def run(i):
        t = sets[i % 2]
        ssm.selective_scan(t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                           dt_bias=t["dt_bias"], ssm_state=t["ssm_state"], slot_idx=t["slot_idx"],
                           out=t["out"], stream=stream)

    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        run(i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    us = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]) * 1e3
    mean = float(us.mean())
    b = W.algorithmic_bytes(spec)["scan"]
    fl = W.chunked_mfma_flops(spec)
    return {"workload": "Mamba-2 prefill, 2 requests x L 4096, 64 heads, headdim 128, dstate 256, "
                        "1 group, bf16 I/O, f32 state to a 1024-slot cache, chunks of 64",
            "us": mean, "us_median": float(np.median(us)),
            "tokens_per_s": spec.batch * spec.seqlen / (mean * 1e-6),
            "bytes": b, "GBps": b / (mean * 1e-6) / 1e9,
            "mfma_flops": fl, "mfma_TFLOPs": fl / (mean * 1e-6) / 1e12,
            "mfma_frac_bf16_peak": fl / (mean * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "kernel_source_sha": kernel_source_sha(KERNEL_SOURCES["chunked_scan"]), "steps": steps}


VARLEN_NSEQ, VARLEN_TOKENS, VARLEN_SEED = 16, 8192, 5


def measure_varlen(ssm, W, dev, stream, steps, warmup):
    """Packed variable-length prefill (continuous batching): 16 sequences of
    mixed lengths, 8192 tokens in all (the token count of the dense prefill),
    every other one continuing from its slot of a 512-slot cache; conv1d
    (the whole call, caches included) then the scan, each timed with events
    on the launch stream over two rotating buffer sets."""
    import numpy as np
    import torch

    lengths = W.varlen_lengths(VARLEN_SEED, VARLEN_NSEQ, VARLEN_TOKENS)
    spec = W.prefill(nslots=512)
    sets = []
    for k in range(2):
        t = W.make_varlen(W.prefill(nslots=512, seed=40 + k), lengths, dev)
        t["u"] = torch.empty_like(t["x"])
        t["out"] = torch.empty_like(t["x"])
        sets.append(t)
    n_init = int(sets[0]["has_init"].sum().item())
    vb = W.varlen_bytes(spec, lengths, n_init)

    def run(i, ev=None):
        t = sets[i % 2]
        if ev is not None:
            ev[0].record(stream)
        ssm.causal_conv1d_varlen(t["x"], t["conv_w"], t["cu_seqlens"], bias=t["conv_b"],
                                 conv_state=t["conv_state"], slot_idx=t["slot_idx"],
                                 has_initial_state=t["has_init"], out=t["u"], stream=stream)
        if ev is not None:
            ev[1].record(stream)
        ssm.selective_scan_varlen(t["u"], t["dt"], t["A"], t["B"], t["C"], t["cu_seqlens"],
                                  D=t["D"], z=t["z"], dt_bias=t["dt_bias"],
                                  ssm_state=t["ssm_state"], slot_idx=t["slot_idx"],
                                  has_initial_state=t["has_init"], out=t["out"], stream=stream)
        if ev is not None:
            ev[2].record(stream)

    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        run(i, ev[i])
    torch.cuda.synchronize()
    per = np.array([[ev[i][0].elapsed_time(ev[i][1]), ev[i][1].elapsed_time(ev[i][2])]
                    for i in range(steps)]).mean(axis=0) * 1e3  # us
    tot_us = per.sum()
    return {
        "workload": f"{VARLEN_NSEQ} packed sequences, {VARLEN_TOKENS} tokens, mixed lengths "
                    "(log-uniform), every other one continuing from its slot; Mamba-1 2.8B "
                    "layer (d_inner 5120, d_state 16, conv 4, f16 io / f32 state)",
        "lengths": lengths,
        "conv1d_varlen": {"bytes": vb["conv"], "us": per[0],
                          "GBps": vb["conv"] / (per[0] * 1e-6) / 1e9,
                          "kernel_source_sha": kernel_source_sha(KERNEL_SOURCES["conv1d_varlen"])},
        "selective_scan_varlen": {"bytes": vb["scan"], "us": per[1],
                                  "GBps": vb["scan"] / (per[1] * 1e-6) / 1e9,
                                  "kernel_source_sha": kernel_source_sha(
                                      KERNEL_SOURCES["selective_scan_varlen"])},
        "GBps": (vb["conv"] + vb["scan"]) / (tot_us * 1e-6) / 1e9,
        "tokens_per_s": VARLEN_TOKENS / (tot_us * 1e-6),
        "steps": steps,
    }


def cpu_baseline(target_s, pspec, dspec):
    """The float64 oracle, as it stands (single thread, plain C), timed on a
    bounded sample of the same step: the prefill (conv1d + scan) of the first
    n channels of request 0, sized to about target_s seconds, plus the whole
    decode step (conv update + state update, 245 requests).  Reported as the
    same algorithmic bytes per second."""
    import numpy as np
    import torch

    import oracle
    import workloads as W

    oracle.build(force=False)
    f = W.to_f64
    t = W.make(pspec, "cpu")
    L, N, Cn = pspec.seqlen, pspec.dstate, pspec.channels

    def run_prefill(nrows):
        # rows are (request, channel) pairs taken request by request
        for b in range(pspec.batch):
            nch = min(Cn, nrows - b * Cn)
            if nch <= 0:
                break
            x = f(t["x"][b:b + 1, :nch])
            u, _, _ = oracle.causal_conv1d(x, f(t["conv_w"][:nch]), f(t["conv_b"][:nch]),
                                           np.zeros((1, nch, 3)), None)
            u = oracle.round_to(u, oracle.F16)
            oracle.selective_scan(u, f(t["dt"][b:b + 1, :nch]), f(t["A"][:nch]),
                                  f(t["B"][b:b + 1]), f(t["C"][b:b + 1]), D=f(t["D"][:nch]),
                                  z=f(t["z"][b:b + 1, :nch]), dt_bias=f(t["dt_bias"][:nch]),
                                  state=np.zeros((1, nch, 1, N)))

    t0 = time.perf_counter()
    run_prefill(32)
    per_ch = (time.perf_counter() - t0) / 32
    d = W.make(dspec, "cpu")
    t0 = time.perf_counter()
    idx = d["slot_idx"].numpy()
    cs = f(d["conv_state"])
    x3 = f(d["x"]).reshape(dspec.batch, dspec.channels, 1)
    u, _, _ = oracle.causal_conv1d(x3, f(d["conv_w"]), f(d["conv_b"]), cs, idx,
                                   has_initial_state=True)
    u = oracle.round_to(u, oracle.F16)
    oracle.state_update(f(d["ssm_state"]), u.reshape(dspec.batch, dspec.nheads, 1), f(d["dt"]),
                        f(d["A"]), f(d["B"]), f(d["C"]), D=f(d["D"]), z=f(d["z"]),
                        dt_bias=f(d["dt_bias"]), slot_idx=idx)
    t_dec = time.perf_counter() - t0
    nch = int(max(32, min(pspec.batch * Cn, (target_s - t_dec) / max(per_ch, 1e-9))))
    t0 = time.perf_counter()
    run_prefill(nch)
    t_pre = time.perf_counter() - t0
    frac = nch / (pspec.batch * pspec.channels)
    pb = W.algorithmic_bytes(pspec)
    db = W.algorithmic_bytes(dspec)
    sample_bytes = frac * (pb["conv"] + pb["scan"]) + db["conv"] + db["ssu"]
    cores = 1
    return {
        "value": sample_bytes / (t_pre + t_dec) / 1e9,
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"prefill conv1d+scan of {nch} of {pspec.batch * pspec.channels} (request, "
                  f"channel) rows at L={L} ({t_pre:.2f} s) + one full decode step, 245 "
                  f"requests ({t_dec:.2f} s); single-threaded float64 C oracle",
        "decode_tokens_per_s": dspec.batch / t_dec,
        "host_cpus_visible": len(os.sched_getaffinity(0)),
        "cpu_model": _cpu_model(),
    }


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
