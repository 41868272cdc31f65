"""Benchmark of the causal selective-SSM hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  prefill  Mamba-1 2.8B layer shape (batch 4, L=2048, d_inner=5120, d_state=16,
           conv width 4, fp16 I/O, fp32 state): causal conv1d + SiLU, then the
           selective scan with the silu(z) gate; final state and conv tail
           written to the cache slots;
  decode   one token for 245 concurrent requests gathered from a 512-slot cache
           (conv cache fp16 [512,5120,3], state cache fp32 [512,5120,16]): the
           conv update fused with the selective state update.
The prefill and decode requests hold separate cache slots, so the step makes
the scan and the decode step in one launch group: they run as one mixed
launch whose decode workgroups follow the scan's and fill the slots its last
round of workgroups leaves free (--serial-step: three separate launches).
Inputs are resident in HBM before the timed region.  Independent buffer sets
are rotated between launches so that no launch re-reads what the previous one
left in the 256 MB Infinity Cache.

Timing follows the benchmark method of the vLLM PR #50534 report (section
"关键源码片段", benchmark_config): launches are captured into one HIP graph,
the graph is replayed a few times untimed, then a number of replays is timed
between two events on the launch stream, and the device time per launch is
the elapsed time over the launch count.  The step is captured as a graph of
10 steps (or the largest divisor of --steps up to 10) and exactly --steps
steps are timed; each kernel is also timed alone (a graph of 10 launches, 5
warm replays, 100 timed replays).

Prints one JSON line.  ``value`` is the whole step's algorithmic HBM traffic
(every input read once, every output written once) divided by the step time,
in GB/s.  Also reported: decode tokens/s at batch 245 (from the decode
kernel's own time), per-kernel GB/s and fraction of the 8 TB/s HBM peak, the
dominant kernel's roofline (its binding resource, the VALU, against the
published FP32 peak, plus its HBM fraction and VALU issue-slot fraction from
the committed counters), a flag per kernel for the 60%-of-HBM target, the
other workloads (the tiny Mamba-1 prefill, the Mamba-2 state updates at
headdim 64 / dstate 128 and headdim 128 / dstate 256 over their batch grids,
the chunked Mamba-2 prefill, the packed variable-length prefill and the whole
decode layer), and the float64 oracle timed on this host's cores (one core,
then all of them) on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import contextlib
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
FP32_PEAK_TFLOPS = 157.3        # MI355X vector FP32, published (counts packed FP32)
# the same units without packed-FP32 forms: 256 CUs x 4 SIMDs x 16 lanes x 2
# flop (FMA) x 2.4 GHz; the kernels here are built without packed FP32
FP32_UNPACKED_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix rate, published
N_SIMD = 256 * 4
N_XCD = 8                       # rocprofv3 reports GRBM_GUI_ACTIVE summed over the XCDs
CLOCK_HZ = 2.4e9
# VALU issue cost of one wave64 instruction in SIMD cycles: 4 for ordinary
# float32 operations; 8 for a float32 transcendental (v_exp_f32 measured at
# half the FMA rate on this chip)
VALU_CYCLES, TRANS_CYCLES = 4, 8
TARGET_HBM_FRAC = 0.60
GRAPH_LAUNCHES, WARM_REPLAYS, TIMED_REPLAYS = 10, 5, 100
ROTATION_BYTES = 512e6          # 2x the Infinity Cache

PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {"selective_scan": ["scan.hip", "scan_body.hpp", "ssm_device.hpp", "ssm_kernels.hpp"],
                  "state_update": ["ssu.hip", "ssu_body.hpp", "ssm_device.hpp", "ssm_kernels.hpp"],
                  "decode_step": ["ssu.hip", "ssu_body.hpp", "ssm_device.hpp", "ssm_kernels.hpp"],
                  "mixed_scan_decode": ["ssu.hip", "scan_body.hpp", "ssu_body.hpp", "ssm_device.hpp",
                                        "ssm_kernels.hpp"],
                  "conv1d_prefill": ["conv1d.hip", "ssm_device.hpp", "ssm_kernels.hpp"],
                  "conv1d_decode": ["conv1d.hip", "ssm_device.hpp", "ssm_kernels.hpp"],
                  "conv1d_varlen": ["conv1d.hip", "ssm_device.hpp", "ssm_kernels.hpp"],
                  "selective_scan_varlen": ["scan.hip", "scan_body.hpp", "ssm_device.hpp", "ssm_kernels.hpp"],
                  "chunked_scan": ["ssd.hip", "ssm_device.hpp", "ssm_kernels.hpp"],
                  "layer_decode": ["gemm.hip", "layer.hip", "conv1d.hip", "ssu.hip", "ssu_body.hpp",
                                   "ssm_device.hpp", "ssm_kernels.hpp"]}
# rocprofv3 kernel names of each headline kernel
KERNEL_SYMBOLS = {"conv1d_prefill": "conv_rows_kernel", "selective_scan": "scan_kernel",
                  "decode_step": "ssu_"}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    # 200 timed steps (about 55 ms) after 50 warm-up steps: a 50-step window
    # right after start-up read 1-2% slow against later windows
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=8.0,
                   help="target duration of each CPU oracle sample (one core, all cores)")
    p.add_argument("--cpu-threads", type=int, default=0,
                   help="threads of the all-core CPU leg (0: every core this process may use)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device copy (for counter calibration)")
    p.add_argument("--ssu-sweep", action="store_true",
                   help="time the Mamba-2 state update over batch, groups and cache dtype "
                        "and print one JSON line per point")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the workloads other than the headline step")
    p.add_argument("--only", choices=["headline", "prefill", "decode", "varlen", "layer", "chunked",
                                      "ssu", "ssu-headline", "tiny"], default=None,
                   help="run one part only (for profiling)")
    p.add_argument("--serial-step", action="store_true",
                   help="launch the step's prefill scan and decode step one after the other "
                        "instead of as one launch group")
    p.add_argument("--unfused-decode", action="store_true",
                   help="decode with the separate conv-update and state-update calls instead "
                        "of the fused decode step")
    p.add_argument("--eager", action="store_true",
                   help="launch eagerly instead of replaying graphs (for counter collection, "
                        "which needs no timing)")
    p.add_argument("--timed-replays", type=int, default=TIMED_REPLAYS)
    p.add_argument("--markers", action="store_true",
                   help="bracket each measurement with a roctx range (for the kernel trace)")
    p.add_argument("--profile-script", metavar="OUTDIR",
                   help="print the rocprofv3 commands whose output --summarize-profile reads")
    p.add_argument("--summarize-profile", metavar="OUTDIR",
                   help="turn rocprofv3 CSV output under OUTDIR into profiles/ summaries")
    return p.parse_args()


def log(msg):
    print(f"bench: {msg}", file=sys.stderr, flush=True)


# --------------------------------------------------------------- markers
_roctx = None


def _roctx_lib():
    global _roctx
    if _roctx is None:
        for name in ("librocprofiler-sdk-roctx.so.1", "/opt/rocm/lib/librocprofiler-sdk-roctx.so.1",
                     "librocprofiler-sdk-roctx.so"):
            try:
                _roctx = ctypes.CDLL(name)
                break
            except OSError:
                continue
        if _roctx is None:
            raise OSError("roctx library not found")
        _roctx.roctxRangePushA.argtypes = [ctypes.c_char_p]
        _roctx.roctxRangePushA.restype = ctypes.c_int
        _roctx.roctxRangePop.argtypes = []
        _roctx.roctxRangePop.restype = ctypes.c_int
    return _roctx


class Marks:
    """roctx ranges around measurements, so that a kernel trace can assign
    every dispatch to the measurement that made it.  The range closes after a
    device synchronisation, so all of its kernels ran inside it."""

    def __init__(self, enabled):
        self.enabled = enabled

    @contextlib.contextmanager
    def __call__(self, label):
        import torch
        if self.enabled:
            torch.cuda.synchronize()
            _roctx_lib().roctxRangePushA(f"bench:{label}".encode())
        try:
            yield
        finally:
            if self.enabled:
                torch.cuda.synchronize()
                _roctx_lib().roctxRangePop()


# ---------------------------------------------------------------- timing
class Timer:
    """Device time per launch of fn(i) (i = launch index, used to rotate
    buffer sets): a graph of `launches` calls, `warm` untimed replays, then
    `timed` replays between two events on the current stream.  With
    eager=True the calls are made directly (counter collection)."""

    def __init__(self, eager=False, timed=TIMED_REPLAYS, warm=WARM_REPLAYS):
        self.eager, self.timed, self.warm = eager, max(1, timed), warm

    def time(self, fn, launches=GRAPH_LAUNCHES, eager_warm=2):
        import torch
        for i in range(eager_warm):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if self.eager:
            e0.record()
            for r in range(self.timed):
                for i in range(launches):
                    fn(i)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / (self.timed * launches)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(launches):
                fn(i)
        for _ in range(self.warm):
            g.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(self.timed):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (self.timed * launches)
        del g
        return us


def kernel_source_sha(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "state_space_model_causal_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _load_profile_json(name, sha):
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != sha:
        return None
    return rec


def load_traffic(kernel: str, sha: str):
    """Counter-measured HBM bytes per launch, if the committed measurement was
    taken on the current kernel source; else None."""
    rec = _load_profile_json(f"{kernel}_traffic.json", sha)
    return None if rec is None else rec.get("hbm_bytes_per_launch")


def valu_issue(counters: dict, us: float) -> dict:
    """VALU issue-slot use of a kernel from its SQ counters (summed over the
    chip, per dispatch): issue cycles the instructions need (4 per wave64
    instruction, 8 per float32 transcendental) over the SIMD cycles
    available, both at the counted clock (the dispatch's GRBM_GUI_ACTIVE
    cycles, which rocprofv3 sums over the 8 XCDs) and at 2.4 GHz over the
    given launch time."""
    insts = counters.get("SQ_INSTS_VALU")
    trans = counters.get("SQ_INSTS_VALU_TRANS_F32", 0.0)
    gui = counters.get("GRBM_GUI_ACTIVE")
    gui = gui / N_XCD if gui else None
    if not insts:
        return None
    need = VALU_CYCLES * (insts - trans) + TRANS_CYCLES * trans
    out = {"valu_insts_per_launch": insts, "trans_f32_insts_per_launch": trans,
           "issue_cycles_needed": need,
           "frac_at_2p4GHz": need / (N_SIMD * CLOCK_HZ * us * 1e-6) if us else None,
           "cost_model": f"{VALU_CYCLES} SIMD cycles per wave64 VALU instruction, "
                         f"{TRANS_CYCLES} per float32 transcendental"}
    if gui:
        out["frac_at_counted_clock"] = need / (N_SIMD * gui)
        out["counted_cycles"] = gui
    if counters.get("SQ_ACTIVE_INST_VALU") and gui:
        # per-SIMD quad-cycles with a VALU instruction in flight, as a share of
        # the dispatch (rocprofiler's VALUBusy: SQ_ACTIVE_INST_VALU / CUs / GUI)
        out["valu_busy"] = counters["SQ_ACTIVE_INST_VALU"] * 4 / (N_SIMD * gui)
    return out


# ------------------------------------------------------------- workloads
def _prefill_sets(W, dev, pspec, n):
    import torch
    sets = []
    for k in range(n):
        t = W.make(W.prefill(seed=pspec.seed + 100 * k), dev)
        t["u"] = torch.empty_like(t["x"])
        t["out"] = torch.empty_like(t["x"])
        sets.append(t)
    return sets


def _decode_sets(W, dev, dspec, n):
    import torch
    sets = []
    for k in range(n):
        t = W.make(W.decode(seed=dspec.seed + 100 * k), dev)
        t["x3"] = t["x"].view(dspec.batch, dspec.channels, 1)
        t["u"] = torch.empty_like(t["x3"])
        t["out"] = torch.empty_like(t["x"])
        sets.append(t)
    return sets


def run_conv_prefill(ssm, t):
    ssm.causal_conv1d(t["x"], t["conv_w"], t["conv_b"], conv_state=t["conv_state"],
                      slot_idx=t["slot_idx"], out=t["u"], has_initial_state=False)


def run_scan_prefill(ssm, t):
    ssm.selective_scan(t["u"], t["dt"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                       dt_bias=t["dt_bias"], ssm_state=t["ssm_state"], slot_idx=t["slot_idx"],
                       has_initial_state=False, out=t["out"])


def run_decode(ssm, t, dspec, fused=True):
    if fused:
        ssm.decode_step(t["ssm_state"], t["conv_state"], t["x"], t["conv_w"], t["dt"], t["A"],
                        t["B"], t["C"], conv_bias=t["conv_b"], D=t["D"], z=t["z"],
                        dt_bias=t["dt_bias"], slot_idx=t["slot_idx"], out=t["out"])
    else:
        ssm.causal_conv1d(t["x3"], t["conv_w"], t["conv_b"], conv_state=t["conv_state"],
                          slot_idx=t["slot_idx"], out=t["u"], has_initial_state=True)
        ssm.state_update(t["ssm_state"], t["u"].view(dspec.batch, dspec.nheads, 1), t["dt"],
                         t["A"], t["B"], t["C"], D=t["D"], z=t["z"], dt_bias=t["dt_bias"],
                         slot_idx=t["slot_idx"], out=t["out"])


def measure_headline(ssm, W, dev, args, timer, mark):
    """The headline step, timed as a graph of steps, and each of its kernels
    timed alone.  Returns (record, host sample of the inputs)."""
    import numpy as np
    import torch

    pspec, dspec = W.prefill(), W.decode()
    pbytes, dbytes = W.algorithmic_bytes(pspec), W.algorithmic_bytes(dspec)
    fused = not args.unfused_decode
    NP = ND = 3  # 3 x ~0.5 GB prefill sets, 3 x ~0.19 GB decode sets
    do_pre = args.only in (None, "headline", "prefill")
    do_dec = args.only in (None, "headline", "decode")
    psets = _prefill_sets(W, dev, pspec, NP) if do_pre else []
    dsets = _decode_sets(W, dev, dspec, ND) if do_dec else []
    torch.cuda.synchronize()
    host = None
    if psets and dsets:
        host = {"prefill": {k: v.cpu() for k, v in psets[0].items()},
                "decode": {k: v.cpu() for k, v in dsets[0].items()}}

    # the prefill's scan and the decode step touch disjoint buffers: made in
    # one launch group they run as one mixed launch (the decode's workgroups
    # after the scan's)
    grouped = bool(psets and dsets and fused and not args.serial_step)

    def step(i):
        if psets:
            run_conv_prefill(ssm, psets[i % NP])
        with (ssm.launch_group() if grouped else contextlib.nullcontext()):
            if psets:
                run_scan_prefill(ssm, psets[i % NP])
            if dsets:
                run_decode(ssm, dsets[i % ND], dspec, fused)

    # the step: W eager warm-up steps, then a graph of G steps replayed
    # (5 warm replays), then exactly K steps timed
    K = args.steps
    G = max(d for d in range(1, min(GRAPH_LAUNCHES, K) + 1) if K % d == 0)
    with mark("step"):
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if args.eager:
            e0.record()
            t_wall0 = time.perf_counter()
            for i in range(K):
                step(i)
        else:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(G):
                    step(i)
            for _ in range(WARM_REPLAYS):
                g.replay()
            torch.cuda.synchronize()
            e0.record()
            t_wall0 = time.perf_counter()
            for _ in range(K // G):
                g.replay()
        e1.record()
        torch.cuda.synchronize()
        t_wall = time.perf_counter() - t_wall0
        ms_per_step = e0.elapsed_time(e1) / K
    log(f"step {ms_per_step * 1e3:.1f} us")

    kernels = {}
    if psets:
        with mark("conv1d_prefill"):
            us = timer.time(lambda i: run_conv_prefill(ssm, psets[i % NP]))
        kernels["conv1d_prefill"] = {"bytes": pbytes["conv"], "us": us}
        with mark("selective_scan"):
            us = timer.time(lambda i: run_scan_prefill(ssm, psets[i % NP]))
        kernels["selective_scan"] = {"bytes": pbytes["scan"], "us": us,
                                     "flops": W.algorithmic_flops(pspec)}
    fused_bytes = dbytes["conv"] + dbytes["ssu"] - 2 * dspec.batch * dspec.channels * 2
    if dsets:
        if fused:
            with mark("decode_step"):
                us = timer.time(lambda i: run_decode(ssm, dsets[i % ND], dspec, True))
            kernels["decode_step"] = {"bytes": fused_bytes, "us": us}
        else:
            with mark("conv1d_decode"):
                us = timer.time(lambda i: ssm.causal_conv1d(
                    dsets[i % ND]["x3"], dsets[i % ND]["conv_w"], dsets[i % ND]["conv_b"],
                    conv_state=dsets[i % ND]["conv_state"], slot_idx=dsets[i % ND]["slot_idx"],
                    out=dsets[i % ND]["u"], has_initial_state=True))
            kernels["conv1d_decode"] = {"bytes": dbytes["conv"], "us": us}
            with mark("state_update"):
                us = timer.time(lambda i: ssm.state_update(
                    dsets[i % ND]["ssm_state"], dsets[i % ND]["u"].view(dspec.batch, dspec.nheads, 1),
                    dsets[i % ND]["dt"], dsets[i % ND]["A"], dsets[i % ND]["B"], dsets[i % ND]["C"],
                    D=dsets[i % ND]["D"], z=dsets[i % ND]["z"], dt_bias=dsets[i % ND]["dt_bias"],
                    slot_idx=dsets[i % ND]["slot_idx"], out=dsets[i % ND]["out"]))
            kernels["state_update"] = {"bytes": dbytes["ssu"], "us": us}
    mixed = None
    if grouped:
        def run_mixed(i):
            with ssm.launch_group():
                run_scan_prefill(ssm, psets[i % NP])
                run_decode(ssm, dsets[i % ND], dspec, True)
        with mark("mixed_scan_decode"):
            us = timer.time(run_mixed)
        mixed = {"us": us, "bytes": pbytes["scan"] + fused_bytes,
                 "GBps": (pbytes["scan"] + fused_bytes) / (us * 1e-6) / 1e9,
                 "kernel_source_sha": kernel_source_sha(KERNEL_SOURCES["mixed_scan_decode"])}
    for k, v in kernels.items():
        v["kernel_source_sha"] = kernel_source_sha(KERNEL_SOURCES[k])
        v["GBps"] = v["bytes"] / (v["us"] * 1e-6) / 1e9
        v["frac_hbm_peak"] = v["GBps"] / HBM_PEAK_GBPS
        v["timing"] = ("eager launches" if args.eager else
                       f"graph of {GRAPH_LAUNCHES} launches, {WARM_REPLAYS} warm + "
                       f"{timer.timed} timed replays")
    log("kernels " + ", ".join(f"{k} {v['us']:.1f} us" for k, v in kernels.items()))

    step_bytes = ((pbytes["conv"] + pbytes["scan"]) if psets else 0) + \
                 ((fused_bytes if fused else dbytes["conv"] + dbytes["ssu"]) if dsets else 0)
    dec_us = (kernels["decode_step"]["us"] if fused else
              kernels["conv1d_decode"]["us"] + kernels["state_update"]["us"]) if dsets else None
    del psets, dsets
    torch.cuda.empty_cache()
    return {"ms_per_step": ms_per_step, "step_graph": G, "wall_s_timed": t_wall,
            "grouped": grouped, "mixed_launch": mixed,
            "step_bytes": step_bytes, "kernels": kernels,
            "decode_us": dec_us, "fused": fused,
            "decode_tokens_per_s": dspec.batch / (dec_us * 1e-6) if dec_us else None,
            "kernel_sum_us": sum(v["us"] for v in kernels.values())}, host


def roofline_of(kernels: dict) -> dict:
    """The dominant kernel's roofline.  The Mamba-1 selective scan is bound by
    float32 VALU issue, not by HBM: per (time, channel, state) element one
    exponential (half-rate) and about six other VALU operations against 0.5
    bytes of HBM traffic.  Its entry carries the FP32 fraction against the
    published 157.3 TFLOP/s, the HBM fraction against 8 TB/s and the VALU
    issue-slot fraction from the committed SQ counters."""
    dom = max(kernels, key=lambda k: kernels[k]["us"])
    dk = kernels[dom]
    sha = kernel_source_sha(KERNEL_SOURCES[dom])
    traffic = load_traffic(dom, sha)
    hbm = {"achieved_GBps": dk["GBps"], "peak_GBps": HBM_PEAK_GBPS, "frac": dk["frac_hbm_peak"],
           "algorithmic_bytes_per_launch": dk["bytes"]}
    if "flops" in dk:
        ach = dk["flops"] / (dk["us"] * 1e-6) / 1e12
        counters = _load_profile_json(f"{dom}_counters.json", sha)
        r = {"kernel": dom, "bound": "alu", "achieved": ach, "peak": FP32_PEAK_TFLOPS,
             "unit": "TFLOP/s", "frac": ach / FP32_PEAK_TFLOPS, "traffic": traffic,
             "flop_model": "per (time, channel, state): delta*A, exp, (delta*u)*B as one op "
                           "each, state and readout FMAs as two each (7); per (time, channel): "
                           "softplus 6, delta*u 1, D*u + add 2, SiLU 4, gate 1 (14)",
             "algorithmic_flops_per_launch": dk["flops"],
             "frac_of_unpacked_fp32": ach / FP32_UNPACKED_TFLOPS,
             "unpacked_fp32_peak": FP32_UNPACKED_TFLOPS,
             "hbm": hbm,
             "valu_issue": valu_issue(counters["counters"], dk["us"]) if counters else None}
    else:
        r = {"kernel": dom, "bound": "hbm", "achieved": dk["GBps"], "peak": HBM_PEAK_GBPS,
             "unit": "GB/s", "frac": dk["frac_hbm_peak"], "traffic": traffic, "hbm": hbm}
    r["algorithmic_bytes_per_launch"] = dk["bytes"]
    r["avg_launch_us"] = dk["us"]
    r["kernel_source_sha"] = sha
    return r


def measure_tiny(ssm, W, dev, timer, mark):
    """The tiny Mamba-1 prefill (batch 1, L 64, d_inner 128, d_state 16,
    f32): conv1d then scan, each timed alone; launch-latency bound."""
    import torch
    spec = W.tiny(nslots=1)
    t = W.make(spec, dev)
    t["u"] = torch.empty_like(t["x"])
    t["out"] = torch.empty_like(t["x"])
    b = W.algorithmic_bytes(spec)
    with mark("tiny_conv1d"):
        cu = timer.time(lambda i: run_conv_prefill(ssm, t))
    with mark("tiny_scan"):
        su = timer.time(lambda i: run_scan_prefill(ssm, t))
    with mark("tiny_pair"):
        pu = timer.time(lambda i: (run_conv_prefill(ssm, t), run_scan_prefill(ssm, t)))
    return {"workload": "Mamba-1 tiny prefill, f32: batch 1, L 64, d_inner 128, d_state 16, "
                        "conv width 4 + SiLU, final state and tail to slot 0",
            "conv1d_us": cu, "scan_us": su, "conv1d_then_scan_us": pu,
            "bytes": b["conv"] + b["scan"], "bound": "launch latency"}


SSU_SHAPES = [
    # (config, name, factory, ngroups, caches, batches, batches the HBM target applies to)
    (3, "m2_ssu_hd64_n128", "m2_ssu_64", (1, 8), ("f16", "f32"), (1, 16, 256, 1024), (256, 1024)),
    (4, "m2_ssu_hd128_n256", "m2_ssu_128", (1,), ("bf16", "f32"), (1, 8, 64, 512), (512,)),
]


def measure_ssu_points(ssm, W, dev, timer, mark, headline_only=False):
    """Mamba-2 state update over batch, ngroups and cache dtype.  Each point
    rotates through disjoint slot sets covering at least 512 MB of cache (so
    no launch finds its state in the on-chip caches) and is timed as graph
    replays of max(10, sets) launches."""
    import torch
    points = []
    for cfg, name, fac, groups, caches, batches, target_batches in SSU_SHAPES:
        factory = getattr(W, fac)
        for G in groups:
            for cache in caches:
                for Bt in batches:
                    if headline_only and Bt != batches[-1]:
                        continue
                    probe = factory(batch=Bt, state=cache, ngroups=G)
                    b = W.algorithmic_bytes(probe)["ssu"]
                    R = max(1, math.ceil(ROTATION_BYTES / b))
                    if probe.random_slots:
                        S = max(probe.slots, Bt * R)
                        spec = factory(batch=Bt, state=cache, ngroups=G, nslots=S)
                        t = W.make(spec, dev)
                        perm = torch.randperm(S, generator=torch.Generator(device=dev).manual_seed(7),
                                              device=dev).to(torch.int32)
                        sets = [perm[r * Bt:(r + 1) * Bt].contiguous() for r in range(R)]
                    else:
                        spec = factory(batch=Bt, state=cache, ngroups=G, nslots=Bt * R)
                        t = W.make(spec, dev)
                        sets = [(torch.arange(Bt, dtype=torch.int32, device=dev) + r * Bt).contiguous()
                                for r in range(R)]
                    out = torch.empty_like(t["x"])

                    def run(i, t=t, out=out, sets=sets, R=R):
                        ssm.state_update(t["ssm_state"], t["x"], t["dt"], t["A"], t["B"], t["C"],
                                         D=t["D"], z=t["z"], dt_bias=t["dt_bias"],
                                         slot_idx=sets[i % R], out=out)

                    label = f"ssu:{name}:g{G}:{cache}:b{Bt}"
                    launches = max(GRAPH_LAUNCHES, R)
                    with mark(label):
                        us = timer.time(run, launches=launches)
                    gbps = b / (us * 1e-6) / 1e9
                    pt = {"config": cfg, "shape": name, "ngroups": G, "cache": cache, "io": spec.io,
                          "batch": Bt, "effective_batch": Bt * spec.nheads, "us": us, "bytes": b,
                          "GBps": gbps, "frac_hbm_peak": gbps / HBM_PEAK_GBPS,
                          "rotation_sets": R, "launches_per_graph": launches, "label": label,
                          "target_batch": Bt in target_batches,
                          "target_met": (gbps / HBM_PEAK_GBPS >= TARGET_HBM_FRAC) if Bt in target_batches else None}
                    log(f"{label}: {us:.1f} us, {gbps:.0f} GB/s")
                    points.append(pt)
                    del t, out, sets
                    torch.cuda.empty_cache()
    return points


def measure_layer(ssm, W, dev, timer, mark):
    """One whole Mamba-1 2.8B decode layer (RMSNorm, in_proj, conv update,
    x_proj, dt_proj, state update, out_proj + residual; random weights) for
    245 requests from a 512-slot cache, f16 I/O and f32 state; two rotating
    sets of caches."""
    import torch

    sets = [W.mamba1_layer(seed=30 + k, device=dev) for k in range(2)]
    descs = [ssm.mamba1_layer(t["w"]) for t in sets]
    lib = ssm.load_library()
    need = lib.ssm_mamba1_decode_layer_workspace(ctypes.byref(descs[0]), 245)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)

    def run(i):
        t = sets[i % 2]
        ssm.mamba1_decode_layer(descs[i % 2], t["hidden"], t["conv_state"], t["ssm_state"],
                                slot_idx=t["slot_idx"], workspace=ws)

    with mark("layer_decode"):
        us = timer.time(run)
    b = W.layer_bytes(2560, 5120, 16, 160, 4, 245)
    return {"workload": "Mamba-1 2.8B decode layer (d_model 2560, d_inner 5120, d_state 16, "
                        "dt_rank 160, conv 4), 245 requests, f16 I/O and weights, f32 state, "
                        "random weights",
            "us": us, "tokens_per_s": 245 / (us * 1e-6),
            "bytes": b["total"], "GBps": b["total"] / (us * 1e-6) / 1e9,
            "frac_hbm_peak": b["total"] / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
            "model_tokens_per_s_64_layers": 245 / (64 * us * 1e-6),
            "kernel_source_sha": kernel_source_sha(KERNEL_SOURCES["layer_decode"])}


def measure_chunked(ssm, W, dev, timer, mark):
    """Mamba-2 prefill in the chunked matrix form (the library's choice for
    bf16 I/O): 2 requests x L 4096, 64 heads of headdim 128, dstate 256,
    bf16 I/O, f32 state written to a 1024-slot cache; two rotating buffer
    sets."""
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
                           out=t["out"])

    with mark("chunked_prefill"):
        us = timer.time(run)
    # the same shape with f16 I/O (also the chunked form)
    del sets[:]
    for k in range(2):
        t = W.make(W.m2_prefill(state="f32", io="f16", seed=spec.seed + 100 * k), dev)
        t["out"] = torch.empty_like(t["x"])
        sets.append(t)
    with mark("chunked_prefill_f16"):
        us16 = timer.time(run)
    # continuous batching: the 8192 tokens as 16 packed sequences of mixed
    # lengths (every other one continuing from its slot), bf16 I/O
    del sets[:]
    lengths = W.varlen_lengths(VARLEN_SEED, VARLEN_NSEQ, VARLEN_TOKENS)
    vspec = W.m2_prefill(state="f32", width=4)
    for k in range(2):
        t = W.make_varlen(W.m2_prefill(state="f32", width=4, seed=spec.seed + 200 + k), lengths, dev)
        t["out"] = torch.empty_like(t["x"])
        sets.append(t)

    def run_packed(i):
        t = sets[i % 2]
        ssm.selective_scan_varlen(t["x"], t["dt"], t["A"], t["B"], t["C"], t["cu_seqlens"], D=t["D"],
                                  z=t["z"], dt_bias=t["dt_bias"], ssm_state=t["ssm_state"],
                                  slot_idx=t["slot_idx"], has_initial_state=t["has_init"], out=t["out"])

    with mark("chunked_prefill_packed"):
        usp = timer.time(run_packed)
    n_init = int(sets[0]["has_init"].sum().item())
    bp = W.varlen_bytes(vspec, lengths, n_init)["scan"]
    del sets[:]
    b = W.algorithmic_bytes(spec)["scan"]
    useful = W.chunked_mfma_flops(spec)
    issued = chunked_issued_mfma_flops(spec)
    issued16 = chunked_issued_mfma_flops(spec, f16_io=True)
    return {"workload": "Mamba-2 prefill, 2 requests x L 4096, 64 heads, headdim 128, dstate 256, "
                        "1 group, bf16 I/O, f32 state to a 1024-slot cache, chunks of 64",
            "us": us, "tokens_per_s": spec.batch * spec.seqlen / (us * 1e-6),
            "bytes": b, "GBps": b / (us * 1e-6) / 1e9,
            "frac_hbm_peak": b / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
            "useful_mfma_flops": useful, "issued_mfma_flops": issued,
            "flop_model": "useful: the chunked form's four products at full chunk x chunk size, "
                          "operands at their own precision (workloads.chunked_mfma_flops); issued: "
                          "the MFMAs the kernel runs (split operands twice, causal tiles skipped, "
                          "the masked decay matrix once per workgroup)",
            "useful_TFLOPs": useful / (us * 1e-6) / 1e12,
            "issued_TFLOPs": issued / (us * 1e-6) / 1e12,
            "useful_frac_bf16_peak": useful / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "issued_frac_bf16_peak": issued / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "f16_io": {"us": us16, "tokens_per_s": spec.batch * spec.seqlen / (us16 * 1e-6),
                       "GBps": b / (us16 * 1e-6) / 1e9,
                       "frac_hbm_peak": b / (us16 * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                       "issued_mfma_flops": issued16,
                       "issued_frac_16bit_peak": issued16 / (us16 * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS},
            "packed": {"workload": f"{VARLEN_NSEQ} packed sequences, {VARLEN_TOKENS} tokens, mixed lengths "
                                   "(log-uniform), every other one continuing from its slot; same heads, "
                                   "bf16 I/O",
                       "lengths": lengths, "us": usp, "tokens_per_s": VARLEN_TOKENS / (usp * 1e-6),
                       "bytes": bp, "GBps": bp / (usp * 1e-6) / 1e9},
            "kernel_source_sha": kernel_source_sha(KERNEL_SOURCES["chunked_scan"])}


def chunked_issued_mfma_flops(spec, chunk=64, rows=64, f16_io=False):
    """Matrix work the chunked Mamba-2 kernel issues, per (request, head, 64
    rows of headdim) workgroup and chunk of 64 steps, in 16x16x32 MFMAs of a
    16-bit type (16384 flops each): C times the carried state, split operand
    (4 step tiles x dstate/32 x 2 x 4 row tiles); the masked C B^T on the 10
    causal tiles of 16 (10 x dstate/32); the state update, split operand
    (dstate/16 x 2 x 2 x 4 row tiles); the outputs, split operand (12 x 4 row
    tiles; with f16 I/O 18 x 4, u being split as well)."""
    N = spec.dstate
    per = 4 * (N // 32) * 2 * 4 + 10 * (N // 32) + (N // 16) * 2 * 2 * 4 + (18 if f16_io else 12) * 4
    wgs = spec.batch * spec.nheads * (spec.headdim // rows)
    chunks = (spec.seqlen + chunk - 1) // chunk
    return float(wgs * chunks * per * 16384)


VARLEN_NSEQ, VARLEN_TOKENS, VARLEN_SEED = 16, 8192, 5


def measure_varlen(ssm, W, dev, timer, mark):
    """Packed variable-length prefill (continuous batching): 16 sequences of
    mixed lengths, 8192 tokens in all (the token count of the dense prefill),
    every other one continuing from its slot of a 512-slot cache; conv1d
    (the whole call, caches included) and the scan, each timed alone over
    two rotating buffer sets."""
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

    def conv(i):
        t = sets[i % 2]
        ssm.causal_conv1d_varlen(t["x"], t["conv_w"], t["cu_seqlens"], bias=t["conv_b"],
                                 conv_state=t["conv_state"], slot_idx=t["slot_idx"],
                                 has_initial_state=t["has_init"], out=t["u"])

    def scan(i):
        t = sets[i % 2]
        ssm.selective_scan_varlen(t["u"], t["dt"], t["A"], t["B"], t["C"], t["cu_seqlens"],
                                  D=t["D"], z=t["z"], dt_bias=t["dt_bias"],
                                  ssm_state=t["ssm_state"], slot_idx=t["slot_idx"],
                                  has_initial_state=t["has_init"], out=t["out"])

    with mark("varlen_conv1d"):
        cu = timer.time(conv)
    with mark("varlen_scan"):
        su = timer.time(scan)
    tot = cu + su
    # the packed scan beside the 245-request decode step of other requests:
    # one after the other, and as one launch group (one mixed launch)
    dspec = W.decode()
    dsets = _decode_sets(W, dev, dspec, 2)

    def serial(i):
        scan(i)
        run_decode(ssm, dsets[i % 2], dspec, True)

    def grouped(i):
        with ssm.launch_group():
            scan(i)
            run_decode(ssm, dsets[i % 2], dspec, True)

    with mark("varlen_scan_decode_serial"):
        ser = timer.time(serial)
    with mark("varlen_scan_decode_grouped"):
        grp = timer.time(grouped)
    del dsets
    return {
        "scan_and_decode_step": {"serial_us": ser, "grouped_us": grp,
                                 "note": "the packed scan and a 245-request decode step from a "
                                         "512-slot cache (other requests), one after the other "
                                         "vs one launch group (one mixed launch)"},
        "workload": f"{VARLEN_NSEQ} packed sequences, {VARLEN_TOKENS} tokens, mixed lengths "
                    "(log-uniform), every other one continuing from its slot; Mamba-1 2.8B "
                    "layer (d_inner 5120, d_state 16, conv 4, f16 io / f32 state)",
        "lengths": lengths,
        "conv1d_varlen": {"bytes": vb["conv"], "us": cu, "GBps": vb["conv"] / (cu * 1e-6) / 1e9,
                          "kernel_source_sha": kernel_source_sha(KERNEL_SOURCES["conv1d_varlen"])},
        "selective_scan_varlen": {"bytes": vb["scan"], "us": su,
                                  "GBps": vb["scan"] / (su * 1e-6) / 1e9,
                                  "kernel_source_sha": kernel_source_sha(
                                      KERNEL_SOURCES["selective_scan_varlen"])},
        "GBps": (vb["conv"] + vb["scan"]) / (tot * 1e-6) / 1e9,
        "tokens_per_s": VARLEN_TOKENS / (tot * 1e-6),
    }


# ---------------------------------------------------------- CPU baseline
def cpu_baseline(target_s, threads, host):
    """The float64 oracle, as it stands (plain sequential C), timed on this
    host on a bounded sample of the same step, from the same bytes the GPU
    received: prefill (conv1d + scan) of whole (request, channel) rows, and
    the decode step (conv update + state update of every request), reported
    as the same algorithmic bytes per second.  First on one core, then on
    `threads` cores: the rows (and for the decode step, channel slices) are
    independent, so a pool of threads each calls the oracle on its own rows
    (the foreign calls release Python's lock, so the threads run in
    parallel)."""
    import concurrent.futures

    import numpy as np

    import oracle
    import workloads as W

    oracle.build(force=False)
    f = W.to_f64
    pspec, dspec = W.prefill(), W.decode()
    p, d = host["prefill"], host["decode"]
    L, N, Cn = pspec.seqlen, pspec.dstate, pspec.channels
    pb, db = W.algorithmic_bytes(pspec), W.algorithmic_bytes(dspec)
    rows_total = pspec.batch * Cn
    x64 = {k: f(p[k]) for k in ("x", "conv_w", "conv_b", "dt", "A", "B", "C", "D", "z", "dt_bias")}

    def prefill_rows(b, c0, c1):
        u, _, _ = oracle.causal_conv1d(x64["x"][b:b + 1, c0:c1], x64["conv_w"][c0:c1],
                                       x64["conv_b"][c0:c1], np.zeros((1, c1 - c0, 3)), None)
        u = oracle.round_to(u, oracle.F16)
        oracle.selective_scan(u, x64["dt"][b:b + 1, c0:c1], x64["A"][c0:c1], x64["B"][b:b + 1],
                              x64["C"][b:b + 1], D=x64["D"][c0:c1], z=x64["z"][b:b + 1, c0:c1],
                              dt_bias=x64["dt_bias"][c0:c1], state=np.zeros((1, c1 - c0, 1, N)))

    def items(nrows, chunk):
        out = []
        for r0 in range(0, nrows, chunk):
            r1 = min(nrows, r0 + chunk)
            b0, b1 = r0 // Cn, (r1 - 1) // Cn
            for b in range(b0, b1 + 1):
                c0 = r0 - b * Cn if b == b0 else 0
                c1 = r1 - b * Cn if b == b1 else Cn
                out.append((b, c0, c1))
        return out

    d64 = {k: f(d[k]) for k in ("conv_state", "x", "conv_w", "conv_b", "ssm_state", "dt", "A", "B",
                                "C", "D", "z", "dt_bias")}
    idx = d["slot_idx"].numpy()

    def decode_slice(c0, c1):
        x3 = d64["x"].reshape(dspec.batch, Cn, 1)[:, c0:c1]
        u, _, _ = oracle.causal_conv1d(x3, d64["conv_w"][c0:c1], d64["conv_b"][c0:c1],
                                       d64["conv_state"][:, c0:c1], idx, has_initial_state=True)
        u = oracle.round_to(u, oracle.F16)
        oracle.state_update(d64["ssm_state"][:, c0:c1], u.reshape(dspec.batch, c1 - c0, 1),
                            d64["dt"][:, c0:c1], d64["A"][c0:c1], d64["B"], d64["C"],
                            D=d64["D"][c0:c1], z=d64["z"][:, c0:c1], dt_bias=d64["dt_bias"][c0:c1],
                            slot_idx=idx)

    # per-row cost on one core, then a sample sized to the target
    t0 = time.perf_counter()
    prefill_rows(0, 0, 32)
    per_row = (time.perf_counter() - t0) / 32
    t0 = time.perf_counter()
    decode_slice(0, Cn)
    t_dec1 = time.perf_counter() - t0
    n1 = int(max(32, min(rows_total, (target_s - t_dec1) / max(per_row, 1e-9))))
    t0 = time.perf_counter()
    for it in items(n1, n1):
        prefill_rows(*it)
    t_pre1 = time.perf_counter() - t0
    b1 = n1 / rows_total * (pb["conv"] + pb["scan"]) + db["conv"] + db["ssu"]
    single = {"value": b1 / (t_pre1 + t_dec1) / 1e9, "unit": "GB/s", "cores": 1,
              "sample": f"prefill conv1d+scan of {n1} of {rows_total} (request, channel) rows at "
                        f"L={L} ({t_pre1:.2f} s) + one full decode step, 245 requests "
                        f"({t_dec1:.2f} s)",
              "decode_tokens_per_s": dspec.batch / t_dec1}

    nt = max(1, threads)
    with concurrent.futures.ThreadPoolExecutor(nt) as ex:
        t0 = time.perf_counter()
        list(ex.map(lambda c: decode_slice(*c),
                    [(c0, min(Cn, c0 + math.ceil(Cn / nt))) for c0 in range(0, Cn, math.ceil(Cn / nt))]))
        t_decn = time.perf_counter() - t0
        nn = int(max(nt * 32, min(rows_total, (target_s - t_decn) * nt * 0.8 / max(per_row, 1e-9))))
        t0 = time.perf_counter()
        list(ex.map(lambda it: prefill_rows(*it), items(nn, 64)))
        t_pren = time.perf_counter() - t0
    bn = nn / rows_total * (pb["conv"] + pb["scan"]) + db["conv"] + db["ssu"]
    return {
        "value": bn / (t_pren + t_decn) / 1e9,
        "unit": "GB/s",
        "cores": nt,
        "kind": "oracle",
        "sample": f"prefill conv1d+scan of {nn} of {rows_total} (request, channel) rows at L={L} "
                  f"({t_pren:.2f} s) + one full decode step, 245 requests ({t_decn:.2f} s); "
                  f"float64 C oracle, {nt} threads over independent rows / channel slices, "
                  "on the same bytes the GPU received",
        "decode_tokens_per_s": dspec.batch / t_decn,
        "single_core": single,
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


# ---------------------------------------------------------------- main
def main():
    args = parse()
    if args.profile_script:
        import bench_profile
        for n, c in bench_profile.profile_commands(args.profile_script):
            print(f'echo "step: {n}" && {c} > {args.profile_script}/{n}.log 2>&1 || exit 1')
        return
    if args.summarize_profile:
        import bench_profile
        bench_profile.summarize_profile(args.summarize_profile)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

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
    mark = Marks(args.markers)
    timer = Timer(eager=args.eager, timed=args.timed_replays)

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
    if args.ssu_sweep:
        for pt in measure_ssu_points(ssm, W, dev, timer, mark):
            print(json.dumps({"ssu_sweep": pt}), flush=True)
        return
    solo = {"layer": ("layer_decode", measure_layer), "chunked": ("chunked_prefill", measure_chunked),
            "varlen": ("varlen_prefill", measure_varlen), "tiny": ("tiny_prefill", measure_tiny)}
    if args.only in solo:
        key, fn = solo[args.only]
        print(json.dumps({key: fn(ssm, W, dev, timer, mark)}), flush=True)
        return
    if args.only in ("ssu", "ssu-headline"):
        pts = measure_ssu_points(ssm, W, dev, timer, mark, headline_only=args.only == "ssu-headline")
        print(json.dumps({"m2_state_update": pts}), flush=True)
        return

    head, host = measure_headline(ssm, W, dev, args, timer, mark)
    kernels = head["kernels"]
    roofline = roofline_of(kernels)
    configs = None
    if not args.no_configs and args.only is None:
        configs = {"tiny_prefill": measure_tiny(ssm, W, dev, timer, mark)}
        configs["m2_state_update"] = measure_ssu_points(ssm, W, dev, timer, mark)
        configs["chunked_prefill"] = measure_chunked(ssm, W, dev, timer, mark)
        log(f"chunked prefill {configs['chunked_prefill']['us']:.1f} us")
        configs["varlen_prefill"] = measure_varlen(ssm, W, dev, timer, mark)
        configs["layer_decode"] = measure_layer(ssm, W, dev, timer, mark)
        log(f"layer {configs['layer_decode']['us']:.1f} us")

    target = {k: v["frac_hbm_peak"] >= TARGET_HBM_FRAC for k, v in kernels.items()
              if k in ("selective_scan", "decode_step", "state_update")}
    if configs:
        for pt in configs["m2_state_update"]:
            if pt["target_batch"]:
                target[pt["label"]] = pt["target_met"]

    cpu = None
    if not args.no_cpu_baseline and host is not None:
        log("cpu baseline")
        thr = args.cpu_threads or len(os.sched_getaffinity(0))
        cpu = cpu_baseline(args.cpu_seconds, thr, host)

    pspec, dspec = W.prefill(), W.decode()
    ms = head["ms_per_step"]
    value = head["step_bytes"] / (ms * 1e-3) / 1e9
    line = {
        "metric": "selective_scan/SSU HBM GB/s + % of roofline; decode tokens/s at batch 245",
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
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
                       "d_state": dspec.dstate, "fused_conv_update": head["fused"]},
            "step_bytes": head["step_bytes"],
            "buffer_sets": {"prefill": 3, "decode": 3},
            "step_launches": ("conv1d; then the scan and the decode step as one mixed launch "
                              "(a launch group: the decode's workgroups after the scan's)"
                              if head["grouped"] else "conv1d, scan, decode step one after the other"),
            "timing": ("eager launches" if args.eager else
                       f"HIP graph of {head['step_graph']} steps, {WARM_REPLAYS} warm replays, "
                       f"{args.steps // head['step_graph']} timed replays"),
            "only": args.only,
        },
        "pct_hbm_roofline": value / HBM_PEAK_GBPS * 100,
        "decode_tokens_per_s": head["decode_tokens_per_s"],
        "kernels": kernels,
        "kernel_sum_us": head["kernel_sum_us"],
        "mixed_launch": head["mixed_launch"],
        "roofline": roofline,
        "target_met": target,
        "cpu_baseline": cpu,
        "configs": configs,
        "wall_s_timed": head["wall_s_timed"],
        "device": props.name,
        "arch": getattr(props, "gcnArchName", None),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
