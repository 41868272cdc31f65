"""rocprofv3 runs behind profiles/, and their summaries.

``python bench.py --profile-script OUT`` prints the commands (run them on the
MI355X from the repository root); ``python bench.py --summarize-profile OUT``
reads their CSV output and writes the summaries under profiles/:

  trace        kernel trace + stats of the whole default benchmark (fewer timed
               replays), with a roctx range around each measurement, so every
               dispatch is attributed to the measurement that made it;
  fetch/write  FETCH_SIZE, then WRITE_SIZE, per dispatch, of the headline
               kernels launched eagerly (one counter per pass);
  ssu_fetch/ssu_write  the same for the Mamba-2 state updates at the largest
               batch of each shape;
  copy_*       the same two counters on a plain 1 GiB device copy, which
               calibrates them to bytes;
  sq           SQ and GRBM counters of the headline kernels (VALU issue of the
               scan, and how much of the conv's and the decode step's time
               their vector work fills);
  ssd          SQ, GRBM and L1->L2 request counters of the chunked Mamba-2
               prefill (matrix-core work, LDS, the B/C stream into the L1s);
  copy_l2      the L1->L2 read requests of the 1 GiB copy (bytes per request).
"""
from __future__ import annotations

import collections
import csv
import glob
import json
import os

import bench

SQ_COUNTERS = ("SQ_WAVES SQ_INSTS_VALU SQ_INSTS_VALU_TRANS_F32 SQ_ACTIVE_INST_VALU SQ_BUSY_CYCLES "
               "SQ_WAVE_CYCLES SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE")
SSD_COUNTERS = ("SQ_WAVES SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_LDS "
                "SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_VALU GRBM_GUI_ACTIVE TCP_TCC_READ_REQ_sum")
HEADLINE_LABELS = {"conv1d_prefill": "conv_rows_kernel", "selective_scan": "scan_kernel",
                   "decode_step": "ssu_", "mixed_scan_decode": "mixed_kernel"}


def profile_commands(out):
    b = "python -u bench.py --no-cpu-baseline"
    pmc = "timeout -s KILL 120 rocprofv3 --pmc {c} -f csv -d {o}/{n} -o run -- {cmd}"
    head = f"{b} --only headline --eager --timed-replays 1 --steps 3 --warmup 1"
    ssu = f"{b} --only ssu-headline --eager --timed-replays 1"
    return [
        ("trace", f"timeout -s KILL 600 rocprofv3 --kernel-trace --marker-trace --stats -f csv "
                  f"-d {out}/trace -o run -- {b} --markers --timed-replays 20 --steps 20 --warmup 5"),
        ("fetch", pmc.format(c="FETCH_SIZE", o=out, n="fetch", cmd=head)),
        ("write", pmc.format(c="WRITE_SIZE", o=out, n="write", cmd=head)),
        ("ssu_fetch", pmc.format(c="FETCH_SIZE", o=out, n="ssu_fetch", cmd=ssu)),
        ("ssu_write", pmc.format(c="WRITE_SIZE", o=out, n="ssu_write", cmd=ssu)),
        ("copy_fetch", pmc.format(c="FETCH_SIZE", o=out, n="copy_fetch",
                                  cmd="python -u bench.py --copy-calibration")),
        ("copy_write", pmc.format(c="WRITE_SIZE", o=out, n="copy_write",
                                  cmd="python -u bench.py --copy-calibration")),
        ("sq", pmc.format(c=SQ_COUNTERS, o=out, n="sq",
                          cmd=f"{b} --only headline --eager --timed-replays 1 --steps 3 --warmup 1")),
        ("ssd", pmc.format(c=SSD_COUNTERS, o=out, n="ssd", cmd=f"{b} --only chunked --eager --timed-replays 1")),
        ("copy_l2", pmc.format(c="TCP_TCC_READ_REQ_sum", o=out, n="copy_l2",
                               cmd="python -u bench.py --copy-calibration")),
    ]


def _one(pattern):
    # rocprofv3 writes under the -d directory, possibly in per-host/per-process
    # subdirectories
    head, tail = os.path.split(pattern)
    g = sorted(glob.glob(pattern)) or sorted(glob.glob(os.path.join(head, "**", tail), recursive=True))
    if not g:
        raise FileNotFoundError(pattern)
    return g[0]


def _rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def _json_line(log, key):
    with open(log) as f:
        for ln in f:
            if ln.startswith("{") and key in ln:
                return json.loads(ln)
    return {}


def _counters(path):
    """{dispatch id: (kernel name, {counter: value})} in dispatch order."""
    out = collections.OrderedDict()
    for r in _rows(path):
        did = int(r.get("Dispatch_Id") or r.get("Correlation_Id") or len(out))
        name = r["Kernel_Name"]
        ent = out.setdefault(did, (name, {}))
        ent[1][r["Counter_Name"]] = ent[1].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def _mean_counters(disp, pred):
    vals = collections.defaultdict(list)
    for name, d in disp.values():
        if pred(name):
            for c, v in d.items():
                vals[c].append(v)
    return {c: sum(v) / len(v) for c, v in vals.items()}, max((len(v) for v in vals.values()), default=0)


def _library(name):
    # kernels launched from graphs are listed under their mangled names
    return "ssm::" in name or name.startswith("_ZN3ssm")


def _markers(path):
    """[(label, start ns, end ns)] of the bench's roctx ranges."""
    ranges = []
    for r in _rows(path):
        lab = None
        for v in r.values():
            if isinstance(v, str) and v.startswith("bench:"):
                lab = v[len("bench:"):]
                break
        if lab is None:
            continue
        ranges.append((lab, int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    return ranges


def _by_marker(trace_rows, ranges):
    """{label: {kernel name: [durations ns]}} for the library's dispatches."""
    out = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in trace_rows:
        name = r["Kernel_Name"]
        if not _library(name):
            continue
        s, e = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        for lab, a, b in ranges:
            if a <= s and e <= b:
                out[lab][name].append(e - s)
                break
    return out


def _stat(durs):
    n = len(durs)
    return n, sum(durs) / n / 1e3, min(durs) / 1e3, max(durs) / 1e3


def _short(name, n=110):
    return name if len(name) <= n else name[:n] + "..."


def summarize_profile(out):
    os.makedirs(bench.PROFILES, exist_ok=True)
    cmds = dict(profile_commands(out))
    import workloads as W

    # calibration of the two traffic counters on a plain device copy
    copy_bytes = 1 << 30
    cf, _ = _mean_counters(_counters(_one(f"{out}/copy_fetch/*counter_collection.csv")),
                           lambda n: "copyBuffer" in n)
    cw, _ = _mean_counters(_counters(_one(f"{out}/copy_write/*counter_collection.csv")),
                           lambda n: "copyBuffer" in n)
    f_factor = copy_bytes / (cf["FETCH_SIZE"] * 1024)
    w_factor = copy_bytes / (cw["WRITE_SIZE"] * 1024)
    calib = (f"Calibration: a plain 1 GiB device copy reads FETCH_SIZE = {cf['FETCH_SIZE']:.0f} KiB "
             f"and WRITE_SIZE = {cw['WRITE_SIZE']:.0f} KiB per dispatch, so HBM bytes = "
             f"FETCH_SIZE x 1024 x {f_factor:.3f} + WRITE_SIZE x 1024 x {w_factor:.3f}.")

    trace_rows = _rows(_one(f"{out}/trace/*kernel_trace.csv"))
    ranges = _markers(_one(f"{out}/trace/*marker_api_trace.csv"))
    bym = _by_marker(trace_rows, ranges)
    line = _json_line(f"{out}/trace.log", '"metric"')
    kern = dict(line.get("kernels", {}))
    if line.get("mixed_launch"):  # the step's scan + decode step as one launch
        kern["mixed_scan_decode"] = line["mixed_launch"]
    cfgs = line.get("configs") or {}

    # ---------------------------------------------------------- headline
    fetch = _counters(_one(f"{out}/fetch/*counter_collection.csv"))
    write = _counters(_one(f"{out}/write/*counter_collection.csv"))
    sq = _counters(_one(f"{out}/sq/*counter_collection.csv"))
    L = ["# Kernel trace, HBM traffic and VALU counters: Mamba-1 2.8B layer step", "",
         "Workload: prefill conv1d+scan, batch 4 x L 2048, d_inner 5120, d_state 16, f16 I/O, "
         "f32 state; one decode step (fused conv update + state update), 245 requests from a "
         "512-slot cache.", "",
         "Commands (run from the repository root on the MI355X):", ""]
    for n in ("trace", "fetch", "write", "copy_fetch", "copy_write", "sq"):
        L.append(f"    {cmds[n]}")
    L += ["", calib, "",
          "Each kernel timed alone (graph replays inside its roctx range `bench:<kernel>`):", "",
          "| kernel | calls | avg us | min us | max us | bench us | algorithmic MB | counter read MB "
          "| counter write MB | traffic / algorithmic |", "|---|---|---|---|---|---|---|---|---|---|"]
    for k, sym in HEADLINE_LABELS.items():
        if k not in bym:
            continue
        durs = [d for nm, ds in bym[k].items() if sym in nm for d in ds]
        n, avg, mn, mx = _stat(durs)
        alg = kern.get(k, {}).get("bytes")
        fr, _ = _mean_counters(fetch, lambda nm: _library(nm) and sym in nm)
        wr, _ = _mean_counters(write, lambda nm: _library(nm) and sym in nm)
        rb = fr.get("FETCH_SIZE", float("nan")) * 1024 * f_factor
        wb = wr.get("WRITE_SIZE", float("nan")) * 1024 * w_factor
        L.append(f"| {k} | {n} | {avg:.1f} | {mn:.1f} | {mx:.1f} | {kern.get(k, {}).get('us', 0):.1f} | "
                 f"{alg / 1e6:.1f} | {rb / 1e6:.1f} | {wb / 1e6:.1f} | {(rb + wb) / alg:.3f} |")
        rec = {"kernel": k, "kernel_source_sha": kern.get(k, {}).get("kernel_source_sha"),
               "fetch_kib_per_dispatch": fr.get("FETCH_SIZE"),
               "write_kib_per_dispatch": wr.get("WRITE_SIZE"),
               "fetch_factor": f_factor, "write_factor": w_factor,
               "hbm_bytes_per_launch": rb + wb, "algorithmic_bytes_per_launch": alg,
               "avg_launch_us_trace": avg, "calls_trace": n,
               "commands": [cmds["fetch"], cmds["write"], cmds["copy_fetch"], cmds["copy_write"]]}
        with open(os.path.join(bench.PROFILES, f"{k}_traffic.json"), "w") as f:
            json.dump(rec, f, indent=1)
    if "step" in bym:
        L += ["", "Inside the graph-replayed step (roctx range `bench:step`; eager warm-up steps "
                  "included):", "", "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
        for nm, ds in bym["step"].items():
            n, avg, mn, mx = _stat(ds)
            L.append(f"| `{_short(nm)}` | {n} | {avg:.1f} | {mn:.1f} | {mx:.1f} |")
    L += ["", f"Bench line of the traced run: step {line.get('ms_per_step', 0) * 1e3:.1f} us, "
              f"{line.get('value', 0):.0f} GB/s, decode {line.get('decode_tokens_per_s', 0) / 1e6:.2f} M "
              "tokens/s."]
    sc, nsc = _mean_counters(sq, lambda nm: _library(nm) and "scan_kernel" in nm)
    scan_sha = kern.get("selective_scan", {}).get("kernel_source_sha")
    scan_us = None
    if "selective_scan" in bym:
        scan_us = _stat([d for ds in bym["selective_scan"].values() for d in ds])[1]
    if sc:
        vi = bench.valu_issue(sc, scan_us)
        L += ["", f"SQ and GRBM counters of the selective scan (mean over {nsc} dispatches; "
                  "command `sq` above):", ""]
        for c in sorted(sc):
            L.append(f"- {c}: {sc[c]:.0f}")
        if sc.get("SQ_WAVES"):
            L.append(f"- VALU instructions per wave: {sc['SQ_INSTS_VALU'] / sc['SQ_WAVES']:.0f}")
        if vi:
            L.append(f"- VALU issue cycles needed ({vi['cost_model']}): {vi['issue_cycles_needed']:.3e}")
            if "frac_at_counted_clock" in vi:
                L.append(f"- as a share of the 1024 SIMDs' cycles during the dispatch "
                         f"(GRBM_GUI_ACTIVE / 8 XCDs = {vi['counted_cycles']:.0f} cycles, "
                         f"{vi['counted_cycles'] / (scan_us * 1e-6) / 1e9 if scan_us else 0:.2f} GHz "
                         f"over the traced time): {vi['frac_at_counted_clock']:.3f}")
            if vi.get("frac_at_2p4GHz"):
                L.append(f"- as a share of 1024 SIMDs x 2.4 GHz x the traced {scan_us:.1f} us: "
                         f"{vi['frac_at_2p4GHz']:.3f}")
            if "valu_busy" in vi:
                L.append(f"- VALU busy (SQ_ACTIVE_INST_VALU x 4 / SIMD cycles): {vi['valu_busy']:.3f}")
        with open(os.path.join(bench.PROFILES, "selective_scan_counters.json"), "w") as f:
            json.dump({"kernel": "selective_scan", "kernel_source_sha": scan_sha,
                       "counters": sc, "dispatches": nsc, "command": cmds["sq"]}, f, indent=1)
    # the other two headline kernels from the same pass: how much of their
    # (memory-bound) time their vector work fills
    others = {}
    for k, sym in (("conv1d_prefill", "conv_rows_kernel"), ("decode_step", "ssu_")):
        oc, noc = _mean_counters(sq, lambda nm, sym=sym: _library(nm) and sym in nm)
        k_us = _stat([d for nm, ds in bym.get(k, {}).items() if sym in nm for d in ds])[1] if k in bym else None
        vi = bench.valu_issue(oc, k_us) if oc else None
        if vi:
            others[k] = {"kernel_source_sha": kern.get(k, {}).get("kernel_source_sha"), "counters": oc,
                         "dispatches": noc, "avg_launch_us_trace": k_us, **vi}
            L.append(f"- {k}: {oc['SQ_INSTS_VALU'] / max(oc.get('SQ_WAVES', 1), 1):.0f} VALU instructions per wave; "
                     f"VALU issue {vi.get('frac_at_counted_clock', float('nan')):.3f} of the SIMD cycles, "
                     f"busy {vi.get('valu_busy', float('nan')):.3f} (mean over {noc} dispatches)")
    if others:
        with open(os.path.join(bench.PROFILES, "headline_valu_counters.json"), "w") as f:
            json.dump({"kernels": others, "command": cmds["sq"]}, f, indent=1)
    _write("mamba1_layer_step_kernels.md", L)

    # --------------------------------------------- Mamba-2 state updates
    pts = cfgs.get("m2_state_update") or []
    sline = _json_line(f"{out}/ssu_fetch.log", "m2_state_update").get("m2_state_update", [])
    sf = _counters(_one(f"{out}/ssu_fetch/*counter_collection.csv"))
    sw = _counters(_one(f"{out}/ssu_write/*counter_collection.csv"))
    traffic = _ssu_traffic(sline, sf, sw, f_factor, w_factor)
    S = ["# Kernel trace and HBM traffic: Mamba-2 state update (configs hd64/N128 and hd128/N256)", "",
         "Each point rotates through disjoint slot sets of at least 512 MB and is replayed as a "
         "graph inside its roctx range `bench:<label>`.", "",
         "Commands (run from the repository root on the MI355X):", "",
         f"    {cmds['trace']}", f"    {cmds['ssu_fetch']}", f"    {cmds['ssu_write']}", "", calib, "",
         "| point | kernel | calls | avg us (trace) | bench us | algorithmic MB | GB/s (trace) | "
         "% of 8 TB/s (trace) | traffic / algorithmic |", "|---|---|---|---|---|---|---|---|---|"]
    recs = []
    for p in pts:
        lab = p["label"]
        if lab not in bym:
            continue
        durs = [d for ds in bym[lab].values() for d in ds]
        names = sorted(bym[lab])
        n, avg, mn, mx = _stat(durs)
        gb = p["bytes"] / (avg * 1e-6) / 1e9
        tr = traffic.get(lab)
        S.append(f"| {lab} | `{_short(names[0], 60)}` | {n} | {avg:.1f} | {p['us']:.1f} | "
                 f"{p['bytes'] / 1e6:.1f} | {gb:.0f} | {gb / bench.HBM_PEAK_GBPS * 100:.1f} | "
                 f"{_ratio(tr, p['bytes'])} |")
        recs.append({"label": lab, "avg_launch_us_trace": avg, "calls_trace": n, "bench_us": p["us"],
                     "algorithmic_bytes_per_launch": p["bytes"], "hbm_bytes_per_launch": tr})
    with open(os.path.join(bench.PROFILES, "mamba2_state_update_traffic.json"), "w") as f:
        json.dump({"kernel_source_sha": bench.kernel_source_sha(bench.KERNEL_SOURCES["state_update"]),
                   "fetch_factor": f_factor, "write_factor": w_factor, "points": recs,
                   "commands": [cmds["trace"], cmds["ssu_fetch"], cmds["ssu_write"]]}, f, indent=1)
    _write("mamba2_state_update_kernels.md", S)

    # ------------------------------------ chunked Mamba-2 prefill counters
    ssd_glob = glob.glob(f"{out}/ssd/**/*counter_collection.csv", recursive=True) + \
        glob.glob(f"{out}/ssd/*counter_collection.csv")
    if ssd_glob:
        cl2, _ = _mean_counters(_counters(_one(f"{out}/copy_l2/*counter_collection.csv")),
                                lambda n: "copyBuffer" in n)
        req_bytes = copy_bytes / cl2["TCP_TCC_READ_REQ_sum"] if cl2.get("TCP_TCC_READ_REQ_sum") else None
        # the dense bf16-I/O prefill: the pass then runs the f16-I/O one and
        # the packed batch (the same bf16 kernel), so only the bf16
        # dispatches in front of the first f16 one are taken
        disp, dense = _counters(ssd_glob[0]), collections.OrderedDict()
        for did, (nm, d) in disp.items():
            if not (_library(nm) and "ssd_kernel" in nm):
                continue
            if not ("ssd_kernel<ssm::bf16" in nm or "ssd_kernelINS_4bf16" in nm):
                break
            dense[did] = (nm, d)
        dc, ndc = _mean_counters(dense, lambda nm: True)
        ch = cfgs.get("chunked_prefill") or {}
        ssd_us = _stat([d for ds in bym.get("chunked_prefill", {}).values() for d in ds])[1] \
            if "chunked_prefill" in bym else None
        flops = dc.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512
        cyc = dc.get("GRBM_GUI_ACTIVE", 0.0) / bench.N_XCD
        l2l1 = dc.get("TCP_TCC_READ_REQ_sum", 0.0) * req_bytes if req_bytes else None
        alg = ch.get("bytes")
        rec = {"kernel": "chunked_prefill (ssd_kernel)",
               "kernel_source_sha": bench.kernel_source_sha(bench.KERNEL_SOURCES["chunked_scan"]),
               "counters": dc, "dispatches": ndc, "avg_launch_us_trace": ssd_us,
               "mfma_flops_per_launch": flops,
               "mfma_tflops_at_trace_time": flops / (ssd_us * 1e-6) / 1e12 if ssd_us else None,
               "frac_of_bf16_dense_peak": flops / (ssd_us * 1e-6) / (bench.MFMA_BF16_PEAK_TFLOPS * 1e12)
               if ssd_us else None,
               "mfma_busy_per_simd_cycle": dc.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (cyc * bench.N_SIMD)
               if cyc else None,
               "valu_busy": dc.get("SQ_ACTIVE_INST_VALU", 0.0) * 4 / (cyc * bench.N_SIMD) if cyc else None,
               "lds_bank_conflict_per_cu_cycle": dc.get("SQ_LDS_BANK_CONFLICT", 0.0) / (cyc * 256) if cyc else None,
               "l1_to_l2_read_bytes": l2l1, "bytes_per_l1_read_request": req_bytes,
               "algorithmic_hbm_bytes": alg,
               "commands": [cmds["ssd"], cmds["copy_l2"], cmds["trace"]]}
        with open(os.path.join(bench.PROFILES, "mamba2_chunked_prefill_counters.json"), "w") as f:
            json.dump(rec, f, indent=1)

    # ----------------------------------------- the other workloads' traces
    for labels, title, fname, rec in (
            (["tiny_conv1d", "tiny_scan", "tiny_pair"], "tiny Mamba-1 prefill (f32, L 64, d_inner 128)",
             "mamba1_tiny_prefill_kernels.md", cfgs.get("tiny_prefill")),
            (["chunked_prefill", "chunked_prefill_f16", "chunked_prefill_packed"],
             "chunked Mamba-2 prefill on MFMA (bf16, f16 I/O, then 16 packed sequences)",
             "mamba2_chunked_prefill_kernels.md",
             cfgs.get("chunked_prefill")),
            (["varlen_conv1d", "varlen_scan"], "packed variable-length prefill (Mamba-1 2.8B layer)",
             "mamba1_varlen_prefill_kernels.md", cfgs.get("varlen_prefill")),
            (["layer_decode"], "whole Mamba-1 2.8B decode layer", "mamba1_decode_layer_kernels.md",
             cfgs.get("layer_decode"))):
        M = [f"# Kernel trace: {title}", "", f"Workload: {(rec or {}).get('workload')}.", "",
             "Command (run from the repository root on the MI355X):", "", f"    {cmds['trace']}", "",
             "| measurement | kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|---|"]
        for lab in labels:
            for nm, ds in bym.get(lab, {}).items():
                n, avg, mn, mx = _stat(ds)
                M.append(f"| {lab} | `{_short(nm, 90)}` | {n} | {avg:.1f} | {mn:.1f} | {mx:.1f} |")
        if rec:
            M += ["", "Bench line of the traced run (graph-replayed device time per call):", "",
                  "```", json.dumps(rec, indent=1), "```"]
        _write(fname, M)


def _ssu_traffic(points, fetch, write, ff, wf):
    """Counter bytes per launch of each eagerly launched state-update point:
    the library's dispatches come in point order, each point making
    2 + launches_per_graph dispatches (two eager warm-ups, one pass)."""
    fd = [(n, d) for n, d in fetch.values() if _library(n)]
    wd = [(n, d) for n, d in write.values() if _library(n)]
    out, i = {}, 0
    for p in points:
        k = 2 + p["launches_per_graph"]
        fs = [d.get("FETCH_SIZE", 0.0) for _, d in fd[i:i + k]]
        ws = [d.get("WRITE_SIZE", 0.0) for _, d in wd[i:i + k]]
        i += k
        if len(fs) == k and len(ws) == k:
            out[p["label"]] = (sum(fs) / k * 1024 * ff) + (sum(ws) / k * 1024 * wf)
    return out


def _ratio(a, b):
    return "" if a is None else f"{a / b:.3f}"


def _write(fname, lines):
    with open(os.path.join(bench.PROFILES, fname), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
