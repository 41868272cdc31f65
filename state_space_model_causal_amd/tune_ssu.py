"""Tune the state update's launch geometry on the GPU and write the gfx950
table (csrc/ssu_table_gfx950.inc) that the library compiles in.

The method follows "[XPU] Add tuned Mamba SSU configs for Intel Arc Pro B70"
(vLLM PR #50534 report, section "实现拆解", steps 2-3): for each key (headdim,
dstate, io dtype, cache dtype) time every candidate geometry over a grid of
effective batches (batch x nheads), and keep a tuned entry only
where the best candidate beats the heuristic by more than 10%; elsewhere the
heuristic stays.  The grid runs to 2M (the Mamba-1 2.8B decode of 245
requests is 1.25M), skipping points whose cache would exceed --max-state-bytes.  The candidates are the geometries ssm_state_update_ex
accepts: 8 or 16 states per lane (also 4 for a float32 cache of at most
256 states per row), workgroups of 64, 128, 256 or 512 lanes.

Each timing captures a HIP graph of launches that rotate through disjoint
slot sets (so repeated launches do not find their state in the on-chip
caches), replays it, and divides the device time by the launch count: the
host's launch rate does not enter.

    python state_space_model_causal_amd/tune_ssu.py --write   # on the GPU

prints one line per measured point, writes a markdown report next to the
table, and (with --write) rewrites the table.  Rebuild the library after.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(_PKG))
import state_space_model_causal_amd as ssm  # noqa: E402

TABLE = os.path.join(_PKG, "csrc", "ssu_table_gfx950.inc")
REPORT = os.path.join(_PKG, "csrc", "ssu_table_gfx950.md")
CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
NAME = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}

# (label, nheads, headdim, dstate, io dtype, cache dtype, one decay per state)
SHAPES = [
    ("mamba1-2.8b", 5120, 1, 16, torch.float16, torch.float32, True),
    ("mamba1-2.8b f16 cache", 5120, 1, 16, torch.float16, torch.float16, True),
    ("mamba2 hd64 n128", 80, 64, 128, torch.float16, torch.float16, False),
    ("mamba2 hd64 n128 f32 cache", 80, 64, 128, torch.float16, torch.float32, False),
    ("mamba2 hd128 n256", 64, 128, 256, torch.bfloat16, torch.bfloat16, False),
    ("mamba2 hd128 n256 f32 cache", 64, 128, 256, torch.bfloat16, torch.float32, False),
]
GRID = [8 << i for i in range(19)]  # effective batch 8 .. 2097152
BLOCKS = (64, 128, 256, 512)


def candidates(dstate, cache):
    """The geometries ssm_state_update_ex accepts for a shape."""
    vs = ((4,) if cache == torch.float32 and dstate <= 256 else ()) + (8, 16)
    return [(v, b) for v in vs for b in BLOCKS]
ADOPT = 0.9  # a tuned geometry must take at most 90% of the heuristic's time


def heuristic(dstate, cache):
    """The library's fallback (ssm.h, ssm_state_update_config): 32 bytes of
    state per lane -- 16 states of a 2-byte cache for rows of >= 32 states
    that are a multiple of 16, else 8 states -- in 256-lane workgroups."""
    two = torch.tensor([], dtype=cache).element_size() == 2
    return (16 if two and dstate % 16 == 0 and dstate >= 32 else 8), 256


def make_inputs(nheads, headdim, dstate, io, cache, a_per_state, batch, ngroups, dev, min_bytes):
    per_req = 2 * nheads * headdim * dstate * torch.tensor([], dtype=cache).element_size()
    rot = max(1, min(64, math.ceil(min_bytes / (batch * per_req))))
    g = torch.Generator(device=dev).manual_seed(1234)
    t = {
        "state": torch.randn(batch * rot, nheads, headdim, dstate, generator=g, device=dev).to(cache),
        "x": torch.randn(batch, nheads, headdim, generator=g, device=dev).to(io),
        "z": torch.randn(batch, nheads, headdim, generator=g, device=dev).to(io),
        "dt": torch.randn(batch, nheads, generator=g, device=dev).to(io),
        "B": torch.randn(batch, ngroups, dstate, generator=g, device=dev).to(io),
        "C": torch.randn(batch, ngroups, dstate, generator=g, device=dev).to(io),
        "dt_bias": torch.rand(nheads, generator=g, device=dev) * -4.0 - 2.0,
        "D": torch.ones(nheads, device=dev),
        "A": (-torch.rand(nheads, dstate, generator=g, device=dev) * 15 - 1 if a_per_state
              else -torch.rand(nheads, generator=g, device=dev) * 15 - 1),
    }
    t["out"] = torch.empty_like(t["x"])
    t["sets"] = [(torch.arange(batch, dtype=torch.int32, device=dev) + r * batch).contiguous()
                 for r in range(rot)]
    return t


def time_config(t, config, launches, replays=5):
    def run(i):
        ssm.state_update(t["state"], t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                         dt_bias=t["dt_bias"], slot_idx=t["sets"][i % len(t["sets"])],
                         out=t["out"], config=config)

    for i in range(3):
        run(i)  # eager warm-up (also validates the config)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(launches):
            run(i)
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (replays * launches)  # us per launch


def tune(shapes, grid, ngroups, min_bytes, max_state_bytes):
    dev = torch.device("cuda:0")
    entries, report = [], []
    for label, H, P, N, io, cache, aps in shapes:
        hv = heuristic(N, cache)
        ssz = torch.tensor([], dtype=cache).element_size()
        batches = sorted({max(1, e // H) for e in grid
                          if max(1, e // H) * H * P * N * ssz <= max_state_bytes})
        prev_eff = 0
        for bi, batch in enumerate(batches):
            eff = batch * H
            t = make_inputs(H, P, N, io, cache, aps, batch, ngroups, dev, min_bytes)
            launches = max(16, len(t["sets"]))
            cands = candidates(N, cache)
            times = {c: time_config(t, c, launches) for c in cands}
            best = min(times, key=times.get)
            adopted = best != hv and times[best] <= ADOPT * times[hv]
            state_bytes = 2 * batch * H * P * N * t["state"].element_size()
            rec = {"shape": label, "batch": batch, "effective_batch": eff,
                   "heuristic": list(hv), "heuristic_us": times[hv], "best": list(best),
                   "best_us": times[best], "adopted": adopted,
                   "state_GBps_best": state_bytes / (times[best] * 1e-6) / 1e9,
                   "all_us": {f"{v}x{b}": times[(v, b)] for v, b in cands}}
            print(json.dumps(rec), flush=True)
            report.append(rec)
            if adopted:
                hi = eff if bi + 1 < len(batches) else (1 << 62)
                entries.append((P, N, CODE[io], CODE[cache], prev_eff, hi, best[0], best[1], label))
            prev_eff = eff
            del t
            torch.cuda.empty_cache()
    return entries, report


def write_table(entries, report, device_name, table=TABLE, report_path=REPORT):
    lines = ["// State-update launch geometry tuned on gfx950 (MI355X); written by",
             "// state_space_model_causal_amd/tune_ssu.py on " + device_name + ", " +
             time.strftime("%Y-%m-%d") + ".  Each line:",
             "// {headdim, dstate, io dtype, cache dtype, effective batch in (lo, hi],"
             " states per lane, workgroup lanes}",
             "// Kept only where the tuned geometry took <= 90% of the heuristic's time."]
    for P, N, io, cache, lo, hi, v, b, label in entries:
        lines.append(f"{{{P}, {N}, {io}, {cache}, {lo}, {hi}, {v}, {b}}},  // {label}")
    with open(table, "w") as f:
        f.write("\n".join(lines) + "\n")
    md = ["# State-update geometry sweep on " + device_name, "",
          "Written by `python state_space_model_causal_amd/tune_ssu.py --write`. Per-launch "
          "device time from graph replays; geometry = states per lane x workgroup lanes; "
          "heuristic = the library's fallback.", "",
          "| shape | batch | effective batch | heuristic | heuristic us | best | best us | "
          "adopted | state GB/s (best) |", "|---|---|---|---|---|---|---|---|---|"]
    for r in report:
        md.append(f"| {r['shape']} | {r['batch']} | {r['effective_batch']} | "
                  f"{r['heuristic'][0]}x{r['heuristic'][1]} | {r['heuristic_us']:.1f} | "
                  f"{r['best'][0]}x{r['best'][1]} | {r['best_us']:.1f} | "
                  f"{'yes' if r['adopted'] else 'no'} | {r['state_GBps_best']:.0f} |")
    with open(report_path, "w") as f:
        f.write("\n".join(md) + "\n")


def main():
    p = argparse.ArgumentParser()
    p.add_argument("--write", action="store_true", help="rewrite the table and the report")
    p.add_argument("--table", default=TABLE, help="where --write puts the table")
    p.add_argument("--report", default=REPORT, help="where --write puts the report")
    p.add_argument("--ngroups", type=int, default=1,
                   help="groups of the timed shapes (use the model's own)")
    p.add_argument("--min-bytes", type=float, default=5e8,
                   help="state bytes each rotation covers (beyond the on-chip caches)")
    p.add_argument("--max-effective-batch", type=int, default=GRID[-1])
    p.add_argument("--max-state-bytes", type=float, default=8e9,
                   help="skip grid points whose state cache would exceed this")
    args = p.parse_args()
    assert torch.cuda.is_available(), "tuning needs the GPU"
    ssm.load_library()
    grid = [e for e in GRID if e <= args.max_effective_batch]
    entries, report = tune(SHAPES, grid, args.ngroups, args.min_bytes, args.max_state_bytes)
    if args.write:
        write_table(entries, report, torch.cuda.get_device_properties(0).name, args.table,
                    args.report)
    print(json.dumps({"adopted_entries": len(entries), "points": len(report)}), flush=True)


if __name__ == "__main__":
    main()
