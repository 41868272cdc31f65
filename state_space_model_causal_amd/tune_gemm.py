"""Sweep the projection kernel's launch plans on the GPU and compare the
library's choice with the best measured one.

The library picks a plan per shape on the host (rows per wave 16/32/64,
64 or 128 columns per workgroup, K splits) from a traffic model of what each
compute unit reads through its L1 (plan_gemm in csrc/gemm.hip).  This tool
times every plan ssm_linear_ex accepts for each shape and reports the
library's plan (ssm_linear_plan), its time, and the best measured plan.

Each timing captures a HIP graph of launches that rotate through enough
copies of the weights (at least --rotate-bytes) that no launch finds its
weights in the on-chip caches, replays it, and divides the device time by
the launch count.

    python state_space_model_causal_amd/tune_gemm.py [--report FILE] [M,N,K ...]

The default shapes are the four projections of the Mamba-1 2.8B decode layer
at 245 requests.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(_PKG))
import state_space_model_causal_amd as ssm  # noqa: E402

LAYER_SHAPES = {"in_proj": (245, 10240, 2560), "x_proj": (245, 192, 5120),
                "dt_proj": (245, 5120, 160), "out_proj": (245, 2560, 5120)}
SPLITS = (1, 2, 3, 4, 5, 6, 8, 10, 12, 16, 20, 24, 32)


def time_plan(x, weights, out, plan, replays):
    """Device time per call of one plan (graph of len(weights) calls)."""
    lib = ssm.load_library()
    M, K = x.shape
    N = weights[0].shape[0]
    wr, c, sp = plan
    need = lib.ssm_linear_workspace_ex(M, N, K, wr, c, sp)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    call = lambda i: ssm.linear(x, weights[i % len(weights)], out=out, workspace=ws, rows_per_wave=wr,
                                cols=c, splits=sp)
    for i in range(2):
        call(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    n = max(10, len(weights))
    with torch.cuda.graph(g):
        for i in range(n):
            call(i)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (replays * n)


def sweep(name, M, N, K, rotate_bytes, replays, dtype=torch.float16):
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(1)
    x = torch.randn(M, K, generator=g, device=dev).to(dtype)
    copies = max(2, math.ceil(rotate_bytes / (N * K * 2)))
    weights = [(torch.randn(N, K, generator=g, device=dev) / K ** 0.5).to(dtype) for _ in range(copies)]
    out = torch.empty(M, N, dtype=dtype, device=dev)
    nb = (K + 63) // 64
    rows = []
    for wr in (16, 32, 64):
        for c in (64, 128):
            for sp in SPLITS:
                if sp > nb:
                    continue
                us = time_plan(x, weights, out, (wr, c, sp), replays)
                rows.append({"plan": [wr, c, sp], "us": us})
                print(json.dumps({"shape": name, "plan": [wr, c, sp], "us": round(us, 2)}), flush=True)
    lib_plan = list(ssm.linear_plan(M, N, K))
    lib_us = next(r["us"] for r in rows if r["plan"] == lib_plan)
    best = min(rows, key=lambda r: r["us"])
    del weights
    torch.cuda.empty_cache()
    return {"shape": name, "M": M, "N": N, "K": K, "library_plan": lib_plan, "library_us": lib_us,
            "best_plan": best["plan"], "best_us": best["us"], "points": rows}


def main():
    p = argparse.ArgumentParser()
    p.add_argument("shapes", nargs="*", help="M,N,K triples (default: the 2.8B decode layer)")
    p.add_argument("--report", help="write a markdown report here")
    p.add_argument("--rotate-bytes", type=float, default=3e8)
    p.add_argument("--replays", type=int, default=50)
    args = p.parse_args()
    shapes = LAYER_SHAPES if not args.shapes else \
        {s: tuple(int(v) for v in s.split(",")) for s in args.shapes}
    results = [sweep(n, *shp, args.rotate_bytes, args.replays) for n, shp in shapes.items()]
    lines = ["# Projection plans on gfx950 (f16, graph-replayed device time per call, reduce included)", "",
             f"Device: {torch.cuda.get_device_name(0)}. Weights rotate through >= {args.rotate_bytes / 1e6:.0f} MB.",
             "", "| shape | M x N x K | library plan (rows/wave, cols, splits) | us | best measured | us | library / best |",
             "|---|---|---|---|---|---|---|"]
    for r in results:
        lines.append(f"| {r['shape']} | {r['M']} x {r['N']} x {r['K']} | {tuple(r['library_plan'])} | "
                     f"{r['library_us']:.1f} | {tuple(r['best_plan'])} | {r['best_us']:.1f} | "
                     f"{r['library_us'] / r['best_us']:.3f} |")
    print("\n".join(lines))
    if args.report:
        with open(args.report, "w") as f:
            f.write("\n".join(lines) + "\n\nEvery plan measured:\n\n")
            for r in results:
                pts = ", ".join(f"{tuple(q['plan'])} {q['us']:.1f}" for q in sorted(r["points"], key=lambda q: q["us"]))
                f.write(f"- {r['shape']}: {pts}\n")


if __name__ == "__main__":
    main()
