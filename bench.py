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
PROFILES = os.path.join(ROOT, "profiles")


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
    p.add_argument("--only", choices=["prefill", "decode"], default=None,
                   help="run only one half of the step (for profiling)")
    return p.parse_args()


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

    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        # ev: list of 5 events bracketing conv, scan, conv update, state update
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

    step_bytes = ((pbytes["conv"] + pbytes["scan"]) if psets else 0) + \
                 ((dbytes["conv"] + dbytes["ssu"]) if dsets else 0)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    def gbps(b, ms):
        return b / (ms * 1e-3) / 1e9 if ms > 0 else None

    kernels = {
        "conv1d_prefill": {"bytes": pbytes.get("conv"), "us": k_ms[0] * 1e3},
        "selective_scan": {"bytes": pbytes.get("scan"), "us": k_ms[1] * 1e3},
        "conv1d_decode": {"bytes": dbytes.get("conv"), "us": k_ms[2] * 1e3},
        "state_update": {"bytes": dbytes.get("ssu"), "us": k_ms[3] * 1e3},
    }
    for v in kernels.values():
        v["GBps"] = gbps(v["bytes"], v["us"] * 1e-3) if v["bytes"] else None
        v["frac_hbm_peak"] = v["GBps"] / HBM_PEAK_GBPS if v["GBps"] else None

    decode_ms = k_ms[2] + k_ms[3]
    decode_tps = dspec.batch / (decode_ms * 1e-3) if dsets else None

    # dominant kernel: the one with the largest share of the step
    dom = max(kernels, key=lambda k: kernels[k]["us"])
    dk = kernels[dom]
    src = {"selective_scan": ["scan.hip", "ssm_device.hpp"],
           "state_update": ["ssu.hip", "ssm_device.hpp"],
           "conv1d_prefill": ["conv1d.hip", "ssm_device.hpp"],
           "conv1d_decode": ["conv1d.hip", "ssm_device.hpp"]}[dom]
    sha = kernel_source_sha(src)
    traffic = load_traffic(dom, sha)
    roofline = {
        "kernel": dom,
        "bound": "hbm",
        "achieved": dk["GBps"],
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": dk["frac_hbm_peak"],
        "traffic": traffic,
        "algorithmic_bytes_per_launch": dk["bytes"],
        "avg_launch_us": dk["us"],
        "kernel_source_sha": sha,
    }

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
                        "d_state 16, conv 4, f16 io / f32 state; + decode conv update + state "
                        "update, 245 requests from a 512-slot cache",
            "prefill": {"batch": pspec.batch, "seqlen": pspec.seqlen, "d_inner": pspec.channels,
                        "d_state": pspec.dstate, "conv_width": pspec.width},
            "decode": {"batch": dspec.batch, "nslots": dspec.nslots, "d_inner": dspec.channels,
                       "d_state": dspec.dstate},
            "step_bytes": step_bytes,
            "buffer_sets": {"prefill": NP, "decode": ND},
            "only": args.only,
        },
        "pct_hbm_roofline": value / HBM_PEAK_GBPS * 100,
        "decode_tokens_per_s": decode_tps,
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "step_ms_median": float(np.median(step_ms)),
        "wall_s_timed": t_wall,
        "device": props.name,
        "arch": getattr(props, "gcnArchName", None),
    }
    print(json.dumps(line), flush=True)


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
    t = W.make(W.prefill(batch=1), "cpu")
    L, N = pspec.seqlen, pspec.dstate

    def run_prefill(nch):
        x = f(t["x"][:, :nch])
        u, _, _ = oracle.causal_conv1d(x, f(t["conv_w"][:nch]), f(t["conv_b"][:nch]),
                                       np.zeros((1, nch, 3)), None)
        u = oracle.round_to(u, oracle.F16)
        oracle.selective_scan(u, f(t["dt"][:, :nch]), f(t["A"][:nch]), f(t["B"]), f(t["C"]),
                              D=f(t["D"][:nch]), z=f(t["z"][:, :nch]),
                              dt_bias=f(t["dt_bias"][:nch]), state=np.zeros((1, nch, 1, N)))

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
    nch = int(max(32, min(pspec.channels, (target_s - t_dec) / max(per_ch, 1e-9))))
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
