"""Benchmark of the SSD hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mamba2_2p7b]

One step = one chunked forward over one batch of the workload: one
ssd_chunked_fwd call through the C ABI (chunk_cumsum, then the one-pass
chunk_state + state_passing stage or the two separate stages -- whichever the
library selects for the shape -- then chunk_scan) on torch's current stream.
The inputs are generated, uploaded and resident in HBM before timing starts;
K steps are timed between two synchronizations and give the tokens/s value.
A second pass runs the same stages one call at a time with HIP events between
them (on the stream the kernels run on) for each kernel's duration, from
which the roofline of the dominant kernel is computed.

Prints one JSON line (stdout): tokens/s of the forward, the roofline of the
dominant kernel, per-kernel times and rooflines, the decode step's HBM
bandwidth on the decode workload, and the CPU oracle's tokens/s on a bounded
sample of the same workload.  Progress goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_mamba2_2p7b.json")
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, published
FP32_VALU_PEAK_TFLOPS = 157.3   # MI355X fp32 vector, published


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---- algorithmic work (what the method must move / compute, per launch) -----------

def algorithmic(w, io_bytes: int, y_bytes: int = 4):
    """Bytes and useful flops each stage must move/compute for workload w.

    Per (b, h, chunk) unit, L tokens, P = 64, N: the bytes each stage must
    read and write once and the flops of its useful products (causal pairs
    only).  B and C are per group and chunk, so their bytes are shared by the
    heads_per_group heads of a group.
    """
    Bt, T, H, P, N, G, L = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk_size
    nc = -(-T // L)
    units = Bt * H * nc
    hpg = H // G
    tok_x = Bt * T * H * P * io_bytes
    tok_bc = Bt * T * G * N * io_bytes
    gdt = 2 * units * L * 4
    state = Bt * H * P * N * 4
    out = {}
    out["chunk_cumsum"] = dict(bytes=Bt * T * H * 4 + gdt, flops=2 * Bt * T * H)
    out["chunk_state"] = dict(bytes=tok_x + tok_bc + gdt + units * P * N * 4,
                              flops=2 * P * N * L * units)
    out["state_passing"] = dict(
        bytes=units * P * N * 4 + units * P * N * io_bytes + units * 4
        + (state if w.init_state else 0) + state,
        flops=2 * units * P * N)
    tri = L * (L + 1) // 2
    tok_y = Bt * T * H * P * y_bytes     # y: fp32, or the io dtype on request
    # one pass: x, B (as MFMA fragments), G and DT in, h_prev out, init/final
    # state; S never exists.  The stage also runs b_fragments (B re-laid out:
    # read once, written once), counted in the stage's bytes.
    out["b_fragments"] = dict(bytes=2 * tok_bc, flops=0)
    # ssd_chunked_fwd builds the fragments in the cumsum's launch
    out["cumsum_bfrag"] = dict(bytes=out["chunk_cumsum"]["bytes"] + out["b_fragments"]["bytes"],
                               flops=out["chunk_cumsum"]["flops"])
    out["state_fwd_kernel"] = dict(
        bytes=tok_x + tok_bc + gdt + units * P * N * io_bytes
        + (state if w.init_state else 0) + state,
        flops=2 * P * N * L * units + 2 * units * P * N)
    out["state_fwd"] = dict(bytes=out["state_fwd_kernel"]["bytes"] + out["b_fragments"]["bytes"],
                            flops=out["state_fwd_kernel"]["flops"])
    out["chunk_scan"] = dict(
        bytes=tok_x + tok_y + 2 * tok_bc + units * P * N * io_bytes + gdt,
        flops=units * (2 * L * P * N + 2 * tri * P) + (Bt * G * nc) * 2 * tri * N)
    # the fused path: one prepass launch (cumsum; B in fp16 fragment order; the
    # causal C B^T tiles in pairs, 16 bytes a lane, 64 lanes per pair of 16x16
    # tiles) and the pass itself (per-group operands counted once)
    nb = L // 16
    cbt = Bt * nc * G * ((nb + 1) // 2) * ((nb + 2) // 2) * 64 * 16
    out["fused_prep"] = dict(bytes=Bt * T * H * 4 + gdt + 3 * tok_bc + cbt,
                             flops=2 * Bt * T * H + (Bt * G * nc) * 2 * tri * N)
    out["fused_fwd"] = dict(
        bytes=tok_x + tok_y + 2 * tok_bc + cbt + gdt + (state if w.init_state else 0) + state,
        flops=units * (4 * L * P * N + 2 * tri * P + 2 * P * N))
    return out


def decode_bytes(w, io_bytes=2):
    Bt, H, P, N, G = w.batch, w.nheads, w.headdim, w.dstate, w.ngroups
    # state read + write, x_t in, y_t out (fp32), dt_t, B_t and C_t
    return (2 * Bt * H * P * N * 4 + Bt * H * P * (io_bytes + 4) + Bt * H * 4
            + 2 * Bt * G * N * io_bytes)


def bwd_bytes(w, io_bytes=2):
    """What the backward must move at least: x, B, C (io dtype), dy, dt, the
    initial state and dfinal (fp32) in; dx, ddt, dB, dC and dinit (fp32) out."""
    Bt, T, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    tok = Bt * T
    ins = tok * H * P * (io_bytes + 4) + 2 * tok * G * N * io_bytes + tok * H * 4
    outs = tok * H * P * 4 + tok * H * 4 + 2 * tok * G * N * 4
    states = 3 * Bt * H * P * N * 4
    return ins + outs + states


def kernel_source_sha(kernel: str) -> str:
    """Hash of the device code a kernel is built from (its .hip file and the
    shared device header; the host-side launch declarations do not enter)."""
    import hashlib
    csrc = os.path.join(ROOT, "selective_state_space_amd", "csrc")
    h = hashlib.sha256()
    files = {"b_fragments": ("state_fwd.hip", "b_fragments.h"),
             "cumsum_bfrag": ("chunk_cumsum.hip", "b_fragments.h"),
             "fused_prep": ("chunk_cumsum.hip", "b_fragments.h", "cb_tiles.h"),
             "fused_fwd": ("fused_fwd.hip", "cb_tiles.h")}.get(kernel, (kernel + ".hip",))
    for f in files + ("ssd_device.h",):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, or None if there is none for this kernel or its source changed since."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    k = rec.get("kernels", {}).get(kernel)
    if not k or rec.get("workload") != workload or k.get("source_sha") != kernel_source_sha(kernel):
        return None
    return int(k["hbm_bytes_per_launch"])


PROFILE_CMD = ("python3 bench.py --forward-only --path=-1,2 --y-dtype both --steps 10 --warmup 3 "
               "--settle-ms 0")
TRACE_CMD = "python3 bench.py --no-cpu-baseline --no-configs"


def profile_kind(name: str):
    """The algorithmic-bytes entry of a forward kernel's (demangled) name; None
    for every other kernel (the gated chunk_scan included)."""
    if "chunk_scan_bf16_kernel" in name:
        # <L, N, GATE, YBF>: the plain forward's launch, with y in fp32 or bf16
        args = [v.strip() for v in name[name.index("<") + 1:name.index(">")].split(",")]
        if args[2] != "false":
            return None
        return "chunk_scan_ybf" if len(args) > 3 and args[3] == "true" else "chunk_scan"
    if "state_fwd_kernel" in name:
        # the forward's mode (bf16 h_prev) only: the backward runs the same
        # kernel with fp32 h_prev (mode 1) and as its adjoint scan (mode 2)
        args = name[name.index("<") + 1:name.index(">")].split(",")
        return "state_fwd_kernel" if args[-1].strip() == "0" else None
    if "fused_fwd_kernel" in name:
        # <L, N, GATE, YBF>, as chunk_scan
        args = [v.strip() for v in name[name.index("<") + 1:name.index(">")].split(",")]
        if args[2] != "false":
            return None
        return "fused_fwd_ybf" if len(args) > 3 and args[3] == "true" else "fused_fwd"
    for k in ("chunk_cumsum", "chunk_state", "state_passing", "b_fragments", "cumsum_bfrag",
              "fused_prep"):
        if k + "_kernel" in name:
            return k
    return None


def summarize_rocprof(pdir: str, workload: str):
    """Writes profiles/kernel_trace_<workload>.md and profiles/traffic_<workload>.{md,json}
    from a rocprofv3 output directory holding trace/ (kernel trace of the
    default bench run), fetch/ and write/ (one counter each over PROFILE_CMD)
    and copyf/ and copyw/ (the same counters over --copy-reference-only)."""
    import collections
    import csv
    import re
    from selective_state_space_amd import inputs as gen

    def short(n):
        n = n.replace("ssd::(anonymous namespace)::", "").replace("void ", "")
        return re.sub(r"\(.*", "", n).replace("unsigned short", "bf16")

    rows = list(csv.DictReader(open(os.path.join(pdir, "trace", "trace_kernel_stats.csv"))))
    out = ["# Kernel trace: %s forward, decode legs and copy reference" % workload, "",
           "Command (from the repo root, on one MI355X):", "",
           "    rocprofv3 --kernel-trace --stats -f csv -d <dir> -o trace -- " + TRACE_CMD, "",
           "| kernel | calls | avg us | min us | max us | % of GPU time |",
           "|---|---|---|---|---|---|"]
    for r in rows:
        out.append("| %s | %s | %.1f | %.1f | %.1f | %s |" % (
            short(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, r["Percentage"]))
    # The same launches split by grid: each leg of the bench (the three
    # forward workloads, the paths, the decode formats) launches a kernel at a
    # grid of its own, so a (kernel, grid) row is one leg's launches.
    tpath = os.path.join(pdir, "trace", "trace_kernel_trace.csv")
    if os.path.exists(tpath):
        groups = collections.defaultdict(list)
        for r in csv.DictReader(open(tpath)):
            key = (short(r["Kernel_Name"]), int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"]),
                   int(r["Workgroup_Size_X"]))
            groups[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        total = sum(sum(v) for v in groups.values())
        out += ["", "The same launches by (kernel, grid): one row per leg's launch shape, rows "
                "above 0.5% of GPU time.", "",
                "| kernel | workgroups x threads | calls | avg us | median us | min us | % of GPU time |",
                "|---|---|---|---|---|---|---|"]
        for (name, nwg, wgs), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
            if sum(v) < 0.005 * total:
                continue
            sv = sorted(v)
            out.append("| %s | %d x %d | %d | %.1f | %.1f | %.1f | %.2f |" % (
                name, nwg, wgs, len(v), sum(v) / len(v), sv[len(sv) // 2], sv[0],
                100.0 * sum(v) / total))
    with open(os.path.join(ROOT, "profiles", "kernel_trace_%s.md" % workload), "w") as fh:
        fh.write("\n".join(out) + "\n")

    def counters(sub):
        agg = collections.defaultdict(list)
        for r in csv.DictReader(open(os.path.join(pdir, sub, sub + "_counter_collection.csv"))):
            agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return agg

    fetch, write = counters("fetch"), counters("write")
    copy_kib = (1 << 30) / 1024
    cf = [v for k, vs in counters("copyf").items() if "copyBuffer" in k for v in vs if v > 1e5]
    cw = [v for k, vs in counters("copyw").items() if "copyBuffer" in k for v in vs if v > 1e5]
    f_fetch, f_write = copy_kib / (sum(cf) / len(cf)), copy_kib / (sum(cw) / len(cw))
    w = gen.BY_NAME[workload]
    io = 2 if w.io_dtype == gen.BF16 else 4
    alg, alg_ybf = algorithmic(w, io), algorithmic(w, io, y_bytes=io)
    res = {"workload": workload,
           "command": "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) -f csv -- " + PROFILE_CMD,
           "copy_calibration": {"bytes_read": 1 << 30, "bytes_written": 1 << 30,
                                "FETCH_SIZE_KiB": sum(cf) / len(cf),
                                "WRITE_SIZE_KiB": sum(cw) / len(cw),
                                "fetch_scale": f_fetch, "write_scale": f_write},
           "kernels": {}}
    md = ["# HBM traffic per launch: %s" % workload, "",
          "Two counter passes of the same bench command (one counter each), from the repo root:",
          "", "    rocprofv3 --pmc FETCH_SIZE -f csv -d <dir> -o fetch -- " + PROFILE_CMD,
          "    rocprofv3 --pmc WRITE_SIZE -f csv -d <dir> -o write -- " + PROFILE_CMD, "",
          "Calibration runs the same two counters over a plain 1 GiB device copy:", "",
          "    rocprofv3 --pmc FETCH_SIZE -f csv -d <dir> -o copyf -- python3 bench.py "
          "--copy-reference-only",
          "    rocprofv3 --pmc WRITE_SIZE -f csv -d <dir> -o copyw -- python3 bench.py "
          "--copy-reference-only", "",
          "The copy (torch `copy_`, the `__amd_rocclr_copyBuffer` kernel) reads %.0f KiB by "
          "FETCH_SIZE and writes %.0f KiB by WRITE_SIZE, so the scale factors are fetch x%.3f and "
          "write x%.3f (1 GiB = 1048576 KiB).  `python3 bench.py --summarize-rocprof <dir>` "
          "wrote this file." % (sum(cf) / len(cf), sum(cw) / len(cw), f_fetch, f_write), "",
          "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes (scaled) | algorithmic bytes "
          "| ratio |", "|---|---|---|---|---|---|"]
    for name in fetch:
        k = profile_kind(name)
        if k is None or name not in write:
            continue
        fk = sum(fetch[name]) / len(fetch[name])
        wk = sum(write[name]) / len(write[name])
        hbm = fk * 1024 * f_fetch + wk * 1024 * f_write
        a = (alg_ybf[k[:-4]]["bytes"] if k.endswith("_ybf") else alg[k]["bytes"])
        src = {"state_fwd_kernel": "state_fwd", "chunk_scan_ybf": "chunk_scan",
               "fused_fwd_ybf": "fused_fwd"}.get(k, k)
        res["kernels"][k] = {"fetch_kib": fk, "write_kib": wk, "hbm_bytes_per_launch": int(hbm),
                             "alg_bytes": a, "source_sha": kernel_source_sha(src)}
        md.append("| %s | %.0f | %.0f | %.4g | %.4g | %.3f |" % (k, fk, wk, hbm, a, hbm / a))
    with open(os.path.join(ROOT, "profiles", "traffic_%s.md" % workload), "w") as fh:
        fh.write("\n".join(md) + "\n")
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(res, fh, indent=1)
    print("\n".join(out))
    print("\n".join(md))


COUNTER_PASSES = (
    "SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_VALU "
    "SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_MISC",
    "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_VMEM_RD "
    "SQ_INSTS_VMEM_WR SQ_LDS_BANK_CONFLICT SQ_WAIT_INST_LDS",
)


def summarize_counters(pdir: str, workload: str):
    """Writes profiles/counters_<workload>.md from rocprofv3 SQ-counter passes:
    <pdir>/{fwd,bwd}{1,2}/c_counter_collection.csv, the passes of COUNTER_PASSES
    over the forward (PROFILE_CMD) and over --backward-only."""
    import collections
    import csv
    import re
    cmds = {"fwd": PROFILE_CMD, "bwd": "python3 bench.py --backward-only"}
    keep = re.compile(r"chunk_scan_bf16_kernel<256, 128, false, (?:false|true)>|"
                      r"state_fwd_kernel<256, 128, 4, [012]>|state_pair_kernel<256, 128, 4>|"
                      r"chunk_cumsum|cumsum_bfrag|fused_prep|"
                      r"fused_fwd_kernel<256, 128, false, (?:false|true)>|bwd_\w+_kernel")
    out = ["# SQ counters per kernel: %s" % workload, "",
           "Two counter passes (rocprofv3 takes at most 8 SQ counters per pass) for each of",
           "the forward and the backward, from the repo root on one MI355X:", ""]
    for leg in ("fwd", "bwd"):
        for i, pas in enumerate(COUNTER_PASSES, 1):
            out.append("    rocprofv3 --pmc %s -f csv -d <dir>/%s%d -o c -- %s" % (pas, leg, i, cmds[leg]))
    out += ["", "Means over the launches of each kernel (the counters sum over the chip;",
            "WAVE_CYCLES and the WAIT/ACTIVE counters are in the same units, so their",
            "ratios are the shares of wave time).  `python3 bench.py --summarize-counters",
            "<dir>` wrote this file.", ""]
    for leg in ("fwd", "bwd"):
        vals = collections.defaultdict(dict)
        for i in (1, 2):
            per = collections.defaultdict(float)
            for r in csv.DictReader(open(os.path.join(pdir, "%s%d" % (leg, i), "c_counter_collection.csv"))):
                per[(r["Kernel_Name"], r["Dispatch_Id"], r["Counter_Name"])] += float(r["Counter_Value"])
            agg = collections.defaultdict(list)
            for (k, d, c), v in per.items():
                agg[(k, c)].append(v)
            for (k, c), vs in agg.items():
                vals[k][c] = sum(vs) / len(vs)
        out += ["## %s" % ("forward" if leg == "fwd" else "backward"), "",
                "| kernel | wave cycles | wait (memory, barrier) | wait (dependency) | VALU issue | "
                "MFMA busy / SIMD | LDS conflict cycles |", "|---|---|---|---|---|---|---|"]
        for k in sorted(vals):
            m = keep.search(k)
            if not m:
                continue
            v = vals[k]
            wc = v.get("SQ_WAVE_CYCLES", 0.0) or 1.0
            name = re.sub(r"\(.*", "", k.replace("ssd::(anonymous namespace)::", "").replace("void ", ""))
            out.append("| %s | %.3g | %.0f%% | %.0f%% | %.0f%% | %.3g | %.3g |" % (
                name.replace("unsigned short", "bf16"), wc, 100 * v.get("SQ_WAIT_ANY", 0) / wc,
                100 * v.get("SQ_WAIT_INST_ANY", 0) / wc, 100 * v.get("SQ_ACTIVE_INST_VALU", 0) / wc,
                v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) / 1024, v.get("SQ_LDS_BANK_CONFLICT", 0)))
        out.append("")
    with open(os.path.join(ROOT, "profiles", "counters_%s.md" % workload), "w") as fh:
        fh.write("\n".join(out) + "\n")
    print("\n".join(out))


# ---- the GPU legs ----------------------------------------------------------------------

def kernel_table(kern, alg):
    """Per-kernel time, bandwidth and fractions of the HBM and bf16 MFMA peaks."""
    out = {}
    for name, ms in kern.items():
        a = alg[name]
        out[name] = dict(
            us=round(ms * 1e3, 2),
            GBps=round(a["bytes"] / (ms * 1e-3) / 1e9, 1),
            hbm_frac=round(a["bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            TFLOPs=round(a["flops"] / (ms * 1e-3) / 1e12, 2),
            bf16_mfma_frac=round(a["flops"] / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            alg_bytes=int(a["bytes"]), alg_flops=int(a["flops"]))
    return out


def _settle(fn, ms: float):
    """Runs fn back to back for about ms milliseconds of wall time (the GPU's
    clocks ramp up over the first few milliseconds of work after idle);
    returns the calls made and the wall time taken."""
    import torch
    n, t0 = 0, time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(4):
            fn()
        n += 4
        torch.cuda.synchronize()
    return n, (time.perf_counter() - t0) * 1e3


STAGES = {
    # ssd_fwd_path -> the stage calls that time that path's kernels, in order
    # (path 1: ssd_state_fwd called alone lays B out itself, work the whole
    # call does inside the cumsum's launch, so its time and bytes include it)
    0: ("chunk_cumsum", "chunk_state", "state_passing", "chunk_scan"),
    1: ("chunk_cumsum", "state_fwd", "chunk_scan"),
}
PATH_NAMES = {0: "four-stage (chunk_state + state_passing)", 1: "one-pass state_fwd",
              2: "fused state and output pass"}


def run_forward(w, steps: int, warmup: int, settle_ms: float = 300.0, path: int = -1,
                y_io: bool = False, stages: bool = True, inp=None):
    """K timed ssd_chunked_fwd calls of workload w (after a clock-settling
    pre-roll and W warm-up calls) on torch's current stream, between two
    synchronizations; each call is also bracketed by HIP events for the
    median and minimum.  With stages, the same path's stage calls are then
    timed one at a time with events between them (the fused path's two
    launches are not separately callable: its stages are left out)."""
    import torch
    from selective_state_space_amd import inputs as gen
    from selective_state_space_amd import ssd

    dev = torch.device("cuda:0")
    t0 = time.time()
    if inp is None:
        inp = gen.make_fwd(w, 0)
    bf = torch.bfloat16 if w.io_dtype == gen.BF16 else torch.float32

    def up(a, dt=torch.float32):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(dev)

    a = ssd.FwdArgs(up(inp.x, bf), up(inp.dt), up(inp.A), up(inp.B, bf), up(inp.C, bf),
                    up(inp.D), w.chunk_size,
                    None if inp.init_state is None else up(inp.init_state), y_io_dtype=y_io)
    log("%s: inputs resident in HBM (%.1f s)" % (w.name, time.time() - t0))
    ssd.set_path_override(path, 0, 0)
    try:
        taken = ssd.fwd_path(a.dims, w.chunk_size)

        def step():
            ssd.ssd_chunked_fwd(a)
        n_settle, settle_wall = _settle(step, settle_ms)
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        t_start = time.perf_counter()
        ev[0].record()
        for k in range(steps):
            step()
            ev[k + 1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
        per_step = np.array([ev[k].elapsed_time(ev[k + 1]) for k in range(steps)])   # ms
        kern = {}
        if stages and taken in (0, 1):
            fns = {"chunk_cumsum": ssd.ssd_chunk_cumsum, "chunk_state": ssd.ssd_chunk_state,
                   "state_passing": ssd.ssd_state_passing, "state_fwd": ssd.ssd_state_fwd,
                   "chunk_scan": ssd.ssd_chunk_scan}
            seq = [(nm, fns[nm]) for nm in STAGES[taken]]
            for _ in range(warmup):
                for _, f in seq:
                    f(a)
            torch.cuda.synchronize()
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(seq) + 1)]
                   for _ in range(steps)]
            for k in range(steps):
                evs[k][0].record()
                for i, (_, f) in enumerate(seq):
                    f(a)
                    evs[k][i + 1].record()
            torch.cuda.synchronize()
            per = np.array([[evs[k][i].elapsed_time(evs[k][i + 1]) for i in range(len(seq))]
                            for k in range(steps)])
            kern = {nm: float(per[:, i].mean()) for i, (nm, _) in enumerate(seq)}
    finally:
        ssd.set_path_override(-1, 0, 0)
    del a
    torch.cuda.empty_cache()
    return dict(wall=wall, mean_ms=float(per_step.mean()), median_ms=float(np.median(per_step)),
                min_ms=float(per_step.min()), kern=kern, path=taken, settle_calls=n_settle,
                settle_ms=round(settle_wall, 1))


def run_decode(w, steps: int, warmup: int, settle_ms: float = 300.0, nset: int = 32):
    """The decode workload's step stream: ``steps`` consecutive steps (512 =
    the workload's length) with the fp32 state carried from step to step,
    every step timed between HIP events.  The per-token inputs are nset
    distinct generated steps used in turn (generating all 512 on the host
    takes ~35 s; they are 0.25% of a step's bytes).  Returns the median,
    mean and minimum milliseconds per step."""
    import torch
    from selective_state_space_amd import inputs as gen
    from selective_state_space_amd import ssd

    dev = torch.device("cuda:0")
    prm = gen.decode_params(w, 0)

    def up(a, dt=torch.float32):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(dev)

    sets = []
    for k in range(nset):
        s = gen.make_decode_step(w, k, prm, 0)
        sets.append((up(s.x_t, torch.bfloat16), up(s.dt_t), up(s.B_t, torch.bfloat16),
                     up(s.C_t, torch.bfloat16)))
    A, D = up(prm.A), up(prm.D)
    state = torch.zeros((w.batch, w.nheads, w.headdim, w.dstate), device=dev)
    y = torch.empty((w.batch, w.nheads, w.headdim), dtype=torch.float32, device=dev)
    _settle(lambda: ssd.ssd_decode_step(state, *sets[0], A, D, y_t=y), settle_ms)
    state.zero_()
    for k in range(warmup):
        ssd.ssd_decode_step(state, *sets[k % nset], A, D, y_t=y)
    state.zero_()   # the stream starts from the zero state
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for k in range(steps):
        ssd.ssd_decode_step(state, *sets[k % nset], A, D, y_t=y)
        ev[k + 1].record()
    torch.cuda.synchronize()
    t = np.array([ev[k].elapsed_time(ev[k + 1]) for k in range(steps)])
    del state
    torch.cuda.empty_cache()
    return float(np.median(t)), float(np.mean(t)), float(np.min(t))


def multi_bytes(w, snapshots: bool, update: bool, io_bytes=2):
    """Algorithmic HBM bytes of one multi-token decode call."""
    Bt, K, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    st = Bt * H * P * N * 4
    tok = Bt * K * (H * P * io_bytes + H * 4 + 2 * G * N * io_bytes + H * P * 4)
    return st * (1 + (K if snapshots else 0) + (1 if update else 0)) + tok


def run_decode_multi(w, steps: int, warmup: int):
    """The multi-token decode workload in its two modes: speculative
    verification (a snapshot after every token, main state not updated) and
    plain multi-token steps (no snapshots, state updated).  Returns the mean
    per-call milliseconds of each."""
    import torch
    from selective_state_space_amd import inputs as gen
    from selective_state_space_amd import ssd

    dev = torch.device("cuda:0")
    prm = gen.decode_params(w, 0)
    m = gen.make_decode_multi(w, prm, 0)
    bf = torch.bfloat16

    def up(a, dt=torch.float32):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(dev)

    args = (up(m.x, bf), up(m.dt), up(m.B, bf), up(m.C, bf), up(prm.A), up(prm.D))
    state = torch.zeros((w.batch, w.nheads, w.headdim, w.dstate), device=dev)
    y = torch.empty((w.batch, w.seqlen, w.nheads, w.headdim), device=dev)
    snaps = torch.empty((w.batch, w.seqlen, w.nheads, w.headdim, w.dstate), device=dev)
    out = {}
    for mode, kw in (("verify", dict(snapshots=snaps, update_state=False)),
                     ("plain", dict(snapshots=None, update_state=True))):
        def call():
            ssd.ssd_decode_multi(state, *args, y=y, **kw)
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            call()
        e1.record()
        torch.cuda.synchronize()
        out[mode] = e0.elapsed_time(e1) / steps
    del state, snaps, y
    torch.cuda.empty_cache()
    return out


def lowp_bytes(w, fmt: str, io_bytes=2):
    """Algorithmic HBM bytes of one decode step on a 16-bit state."""
    Bt, H, P, N, G = w.batch, w.nheads, w.headdim, w.dstate, w.ngroups
    st = Bt * H * P * N * 2 * 2 + (Bt * H * P * 4 * 2 if fmt == "int16" else 0)
    return st + Bt * (H * P * io_bytes + H * 4 + 2 * G * N * io_bytes + H * P * 4)


def run_decode_lowp(w, steps: int, warmup: int):
    """The decode step on decode_b256 with the state stored at 16 bits:
    median per-step milliseconds for each format."""
    import torch
    from selective_state_space_amd import inputs as gen
    from selective_state_space_amd import ssd

    dev = torch.device("cuda:0")
    prm = gen.decode_params(w, 0)
    s = gen.make_decode_step(w, 0, prm, 0)

    def up(a, dt=torch.float32):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(dev)

    args = (up(s.x_t, torch.bfloat16), up(s.dt_t), up(s.B_t, torch.bfloat16),
            up(s.C_t, torch.bfloat16), up(prm.A), up(prm.D))
    y = torch.empty((w.batch, w.nheads, w.headdim), dtype=torch.float32, device=dev)
    out = {}
    for name, fmt, stoch in (("f16", "f16", False), ("f16_stochastic", "f16", True),
                             ("bf16", "bf16", False), ("int16", "int16", False)):
        state = torch.zeros((w.batch, w.nheads, w.headdim, w.dstate),
                            dtype=ssd.STATE_DTYPES[fmt][1], device=dev)
        scale = (torch.zeros((w.batch, w.nheads, w.headdim), device=dev) if fmt == "int16"
                 else None)
        for k in range(warmup):
            ssd.ssd_decode_step_lp(state, *args, fmt, scale=scale, philox_rounds=10 * stoch, seed=k, y_t=y)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record()
        for k in range(steps):
            ssd.ssd_decode_step_lp(state, *args, fmt, scale=scale, philox_rounds=10 * stoch, seed=k, y_t=y)
            ev[k + 1].record()
        torch.cuda.synchronize()
        out[name] = float(np.median([ev[k].elapsed_time(ev[k + 1]) for k in range(steps)]))
        del state, scale
    torch.cuda.empty_cache()
    return out


def run_backward(w, steps: int, warmup: int):
    """ssd_chunked_bwd on the forward workload (dy ~ N(0,1), dfinal ~ N(0,1));
    mean milliseconds per call over ``steps`` calls."""
    import torch
    from selective_state_space_amd import inputs as gen
    from selective_state_space_amd import ssd

    dev = torch.device("cuda:0")
    inp = gen.make_fwd(w, 0)
    bf = torch.bfloat16 if w.io_dtype == gen.BF16 else torch.float32

    def up(a, dt=torch.float32):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(dev)

    rng = np.random.default_rng(9)
    args = (up(inp.x, bf), up(inp.dt), up(inp.A), up(inp.B, bf), up(inp.C, bf), up(inp.D),
            w.chunk_size, up(rng.standard_normal(inp.x.shape, dtype=np.float32)),
            None if inp.init_state is None else up(inp.init_state),
            up(rng.standard_normal((w.batch, w.nheads, w.headdim, w.dstate), dtype=np.float32)))
    del inp
    a = ssd.FwdArgs(*args[:7], init_state=args[8])
    ws = torch.empty(ssd.ssd_chunked_bwd_workspace_size(a.dims, w.chunk_size), dtype=torch.uint8,
                     device=dev)
    del a
    _settle(lambda: ssd.ssd_chunked_bwd(*args, workspace=ws), 300.0)
    for _ in range(warmup):
        ssd.ssd_chunked_bwd(*args, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        ssd.ssd_chunked_bwd(*args, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del args, ws
    torch.cuda.empty_cache()
    return ms


def run_layer_interface(w, wd, steps: int, warmup: int):
    """The forward and decode step with every layer option on (dt_bias,
    softplus, the z gate).  The raw steps are the inverse softplus of the
    workload's dt with a zero bias, so the recurrence sees the same steps as
    the plain run; z is standard normal in x's dtype."""
    import torch
    from selective_state_space_amd import inputs as gen
    from selective_state_space_amd import ssd

    dev = torch.device("cuda:0")

    def up(a, dt=torch.float32):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(dev)

    def inv_softplus(d):
        d = np.asarray(d, np.float64)
        return np.log(np.expm1(d)).astype(np.float32)

    def timed(fn, n, k0):
        _settle(fn, 300.0)
        for _ in range(k0):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    bf = torch.bfloat16 if w.io_dtype == gen.BF16 else torch.float32
    inp = gen.make_fwd(w, 0)
    rng = np.random.default_rng(3)
    z = up(rng.standard_normal(inp.x.shape, dtype=np.float32), bf)
    a = ssd.FwdArgs(up(inp.x, bf), up(inv_softplus(inp.dt)), up(inp.A), up(inp.B, bf),
                    up(inp.C, bf), up(inp.D), w.chunk_size,
                    None if inp.init_state is None else up(inp.init_state),
                    dt_bias=torch.zeros(w.nheads, device=dev), dt_softplus=True, z=z)
    del inp
    fwd_ms = timed(lambda: ssd.ssd_chunked_fwd(a), steps, warmup)
    del a, z
    torch.cuda.empty_cache()

    prm = gen.decode_params(wd, 0)
    s = gen.make_decode_step(wd, 0, prm, 0)
    state = torch.zeros((wd.batch, wd.nheads, wd.headdim, wd.dstate), device=dev)
    y = torch.empty((wd.batch, wd.nheads, wd.headdim), dtype=torch.float32, device=dev)
    zt = up(rng.standard_normal(s.x_t.shape, dtype=np.float32), torch.bfloat16)
    args = (up(s.x_t, torch.bfloat16), up(inv_softplus(s.dt_t)), up(s.B_t, torch.bfloat16),
            up(s.C_t, torch.bfloat16), up(prm.A), up(prm.D))
    bias = torch.zeros(wd.nheads, device=dev)
    dec_ms = timed(lambda: ssd.ssd_decode_step(state, *args, y_t=y, dt_bias=bias,
                                               dt_softplus=True, z_t=zt), 50, 5)
    del state
    torch.cuda.empty_cache()
    return fwd_ms, dec_ms


def run_copy_reference(nbytes: int = 1 << 30, reps: int = 10):
    """HBM bandwidth of torch's device copy (read + write), for context."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1.0)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    torch.cuda.empty_cache()
    return 2 * nbytes / (ms * 1e-3) / 1e9


# ---- the CPU baseline: the oracle on a bounded sample ------------------------------------

def run_cpu_baseline(w, target_s: float = 12.0):
    import oracle
    from selective_state_space_amd import inputs as gen

    inp = gen.make_fwd(w, 0)
    Bt, H = w.batch, w.nheads
    npairs_all = Bt * H
    rng = np.random.default_rng(1)
    order = rng.permutation(npairs_all)
    # calibrate on a few pairs, then size the sample to about target_s seconds
    k = min(16, npairs_all)
    t0 = time.perf_counter()
    _, _, nth = oracle.token_fwd(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.init_state,
                                 pairs=sorted(order[:k]))
    t_cal = time.perf_counter() - t0
    per_pair = t_cal / k
    k2 = int(min(npairs_all, max(k, target_s / max(per_pair, 1e-9))))
    k2 = max(nth, (k2 // nth) * nth) if k2 > nth else k2
    # where the whole job takes less than target_s, it is run again (at most
    # 20 passes) so that the timing covers about target_s of CPU work
    reps = int(min(20, max(1, round(target_s / max(per_pair * k2, 1e-9))))) if k2 == npairs_all else 1
    t0 = time.perf_counter()
    for _ in range(reps):
        _, _, nth = oracle.token_fwd(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.init_state,
                                     pairs=sorted(order[:k2]))
    t = time.perf_counter() - t0
    frac = k2 / npairs_all
    tokens = Bt * w.seqlen * frac * reps   # the sampled share of the whole job's tokens
    return dict(value=tokens / t, unit="tokens/s", cores=int(nth), kind="oracle",
                sample="float64 token recurrence over %d of the %d (batch, head) pairs, all %d "
                       "tokens each (%.1f%% of the job), %d pass(es), %.2f s wall; value = "
                       "sampled tokens / wall time" % (k2, npairs_all, w.seqlen, 100 * frac, reps,
                                                       t))


# ---- main ----------------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="mamba2_2p7b")
    ap.add_argument("--decode-steps", type=int, default=512)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the 370M and long-context forward legs and the path comparison")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="clock-settling pre-roll before each leg's counted warm-up (ms of "
                         "back-to-back calls)")
    ap.add_argument("--summarize-rocprof", metavar="DIR",
                    help="write the profiles/ summaries from a rocprofv3 output directory "
                         "(host only, no GPU)")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="write profiles/counters_<workload>.md from SQ-counter passes (host only)")
    ap.add_argument("--backward-only", action="store_true",
                    help="only the backward leg (for profiling): prints its mean time per call")
    ap.add_argument("--forward-only", action="store_true",
                    help="only the forward leg of --workload (for profiling): prints its median "
                         "time per call; --path picks the forward path (-1 = the default)")
    ap.add_argument("--path", default="-1",
                    help="forward path(s) for --forward-only, comma-separated ssd_fwd_path "
                         "values (-1 = the default)")
    ap.add_argument("--y-dtype", choices=("f32", "io", "both"), default="f32",
                    help="--forward-only: y in fp32, in the io dtype, or one leg of each")
    ap.add_argument("--copy-reference-only", action="store_true",
                    help="only the 1 GiB device copy (calibrates HBM byte counters)")
    args = ap.parse_args()

    if args.summarize_rocprof:
        summarize_rocprof(args.summarize_rocprof, args.workload)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.workload)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only (a single MI355X; there is no multi-GPU "
              "path): run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from selective_state_space_amd import inputs as gen
    from selective_state_space_amd import ssd

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_reference_only:
        print(json.dumps({"hbm_copy_reference_GBps": round(run_copy_reference(), 1),
                          "bytes_read": 1 << 30, "bytes_written": 1 << 30}), flush=True)
        return
    ssd.load_library()   # fails loudly if libssd.so is missing

    w = gen.BY_NAME[args.workload]
    if args.forward_only:
        inp = gen.make_fwd(w, 0)
        yio = {"f32": (False,), "io": (True,), "both": (False, True)}[args.y_dtype]
        for pth, yi in ((int(v), yi) for v in args.path.split(",") for yi in yio):
            r = run_forward(w, args.steps, args.warmup, args.settle_ms, path=pth,
                            y_io=yi, stages=False, inp=inp)
            print(json.dumps({"workload": w.name, "path": PATH_NAMES[r["path"]],
                              "y_io_dtype": yi,
                              "median_us_per_call": round(r["median_ms"] * 1e3, 2),
                              "min_us_per_call": round(r["min_ms"] * 1e3, 2)}), flush=True)
        return
    if args.backward_only:
        bms = run_backward(w, 10, 10)
        print(json.dumps({"workload": w.name, "backward_us_per_call": round(bms * 1e3, 2)}),
              flush=True)
        return
    io_bytes = 2 if w.io_dtype == gen.BF16 else 4
    log("workload %s: %s" % (w.name, w.description))

    inp = gen.make_fwd(w, 0)
    fw = run_forward(w, args.steps, args.warmup, args.settle_ms, inp=inp)
    wall, kern = fw["wall"], fw["kern"]
    step_ms = wall / args.steps * 1e3
    tokens = w.batch * w.seqlen
    value = tokens * args.steps / wall
    alg = algorithmic(w, io_bytes)
    kernels = kernel_table(kern, alg)
    dom = max(kern, key=kern.get)
    dms = kern[dom]
    achieved = alg[dom]["bytes"] / (dms * 1e-3) / 1e9
    # the same launch against the byte count with y stored in the io dtype
    # (what the pages' interfaces return): the bf16 y store is a third of
    # chunk_scan's bytes smaller
    alg_yio = algorithmic(w, io_bytes, y_bytes=io_bytes)
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": measured_traffic(dom, w.name),
                "avg_launch_us": round(dms * 1e3, 2), "alg_bytes_per_launch": int(alg[dom]["bytes"]),
                "alg_bytes_per_launch_y_io_dtype": int(alg_yio[dom]["bytes"]),
                "frac_y_io_dtype_bytes": round(alg_yio[dom]["bytes"] / (dms * 1e-3) / 1e9
                                               / HBM_PEAK_GBPS, 4)}
    mfma_kernels = [k for k in ("chunk_state", "state_fwd", "chunk_scan") if k in kern]
    chunk_flops = sum(alg[k]["flops"] for k in mfma_kernels)
    chunk_ms = sum(kern[k] for k in mfma_kernels)
    fwd_flops = sum(alg[k]["flops"] for k in kern)
    log("forward: %.1f us/step (wall; median %.1f, min %.1f), %.3e tokens/s; stages %s"
        % (step_ms * 1e3, fw["median_ms"] * 1e3, fw["min_ms"] * 1e3, value,
           " ".join("%s %.1f" % (k, v * 1e3) for k, v in kern.items())))

    # y in the io dtype (bf16): the same call with ssd_layer_opts.y_io_dtype.
    # The stage calls take no options (their y is float32), so chunk_scan's
    # time with bf16 stores is the whole call less the other two stages of
    # the leg above (rocprofv3's kernel trace gives it directly)
    fy = run_forward(w, args.steps, args.warmup, args.settle_ms, y_io=True, stages=False, inp=inp)
    yio_us = fy["median_ms"] * 1e3
    scan_us = yio_us - sum(v for k, v in kern.items() if k != "chunk_scan") * 1e3
    y_io = dict(us=round(fy["wall"] / args.steps * 1e6, 2),
                median_us=round(yio_us, 2), min_us=round(fy["min_ms"] * 1e3, 2),
                tokens_per_s=round(tokens * args.steps / fy["wall"], 1),
                y_bytes_saved=int(alg["chunk_scan"]["bytes"] - alg_yio["chunk_scan"]["bytes"]),
                chunk_scan_us_by_difference=round(scan_us, 2),
                chunk_scan_hbm_frac_by_difference=round(
                    alg_yio["chunk_scan"]["bytes"] / (scan_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4))
    log("forward, bf16 y: %.1f us/step (median %.1f); chunk_scan ~%.1f us"
        % (y_io["us"], yio_us, scan_us))

    # every path on this workload, then the other forward configurations
    paths = {}
    for pth in (0, 1, 2):
        if pth == fw["path"]:
            r = fw
        else:
            r = run_forward(w, max(10, args.steps // 2), args.warmup, args.settle_ms, path=pth,
                            stages=False, inp=inp)
        paths[PATH_NAMES[r["path"]]] = dict(median_us=round(r["median_ms"] * 1e3, 2),
                                           min_us=round(r["min_ms"] * 1e3, 2))
    log("paths: " + ", ".join("%s %.1f us" % (k, v["median_us"]) for k, v in paths.items()))
    del inp
    configs = {w.name: dict(tokens_per_s=round(value, 1), median_us=round(fw["median_ms"] * 1e3, 2),
                            path=PATH_NAMES[fw["path"]], paths=paths)}
    if not args.no_configs:
        for idx, (nsteps, nwarm) in ((1, (args.steps, args.warmup)), (3, (10, 3))):
            wc = gen.WORKLOADS[idx]
            if wc.name == w.name:
                continue
            ic = gen.make_fwd(wc, 0)
            rc = run_forward(wc, nsteps, nwarm, args.settle_ms, inp=ic)
            ac = algorithmic(wc, 2 if wc.io_dtype == gen.BF16 else 4)
            kc = kernel_table(rc["kern"], ac)
            cflops = sum(ac[k]["flops"] for k in rc["kern"])
            cp = {PATH_NAMES[rc["path"]]: dict(median_us=round(rc["median_ms"] * 1e3, 2),
                                                min_us=round(rc["min_ms"] * 1e3, 2))}
            for pth in (0, 1, 2):
                if pth != rc["path"]:
                    r = run_forward(wc, nsteps, nwarm, args.settle_ms, path=pth, stages=False,
                                    inp=ic)
                    cp[PATH_NAMES[r["path"]]] = dict(median_us=round(r["median_ms"] * 1e3, 2),
                                                     min_us=round(r["min_ms"] * 1e3, 2))
            del ic
            configs[wc.name] = dict(
                tokens=wc.batch * wc.seqlen,
                us=round(rc["wall"] / nsteps * 1e6, 2), median_us=round(rc["median_ms"] * 1e3, 2),
                min_us=round(rc["min_ms"] * 1e3, 2),
                tokens_per_s=round(wc.batch * wc.seqlen * nsteps / rc["wall"], 1),
                steps=nsteps, warmup=nwarm, path=PATH_NAMES[rc["path"]], kernels=kc,
                forward_bf16_mfma_frac=round(cflops / (rc["median_ms"] * 1e-3) / 1e12
                                             / BF16_PEAK_TFLOPS, 4),
                paths=cp)
            log("%s: %.1f us/call (median), %.3e tokens/s; %s" % (
                wc.name, rc["median_ms"] * 1e3, configs[wc.name]["tokens_per_s"],
                ", ".join("%s %.1f" % (k, v["median_us"]) for k, v in cp.items())))

    decode = None
    if not args.no_decode:
        wd = gen.WORKLOADS[4]
        med, mean, mn = run_decode(wd, args.decode_steps, 5, args.settle_ms)
        byt = decode_bytes(wd)
        decode = dict(workload=wd.name, us_per_step=round(med * 1e3, 2),
                      mean_us=round(mean * 1e3, 2), min_us=round(mn * 1e3, 2),
                      GBps=round(byt / (med * 1e-3) / 1e9, 1),
                      hbm_frac=round(byt / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                      tokens_per_s=round(wd.batch / (med * 1e-3), 1),
                      alg_bytes_per_step=int(byt), steps_timed=args.decode_steps,
                      inputs="%d consecutive steps, state carried, 32 generated input sets in turn"
                             % args.decode_steps)
        log("decode: %.1f us/step, %.0f GB/s" % (med * 1e3, decode["GBps"]))
    multi = None
    if not args.no_decode:
        wm = gen.BY_NAME["mtp_verify_b256_k4"]
        ms = run_decode_multi(wm, 20, 5)
        multi = {"workload": wm.name, "tokens_per_call": wm.batch * wm.seqlen}
        for mode, snap, upd in (("verify", True, False), ("plain", False, True)):
            byt = multi_bytes(wm, snap, upd)
            multi[mode] = dict(us_per_call=round(ms[mode] * 1e3, 2),
                               tokens_per_s=round(wm.batch * wm.seqlen / (ms[mode] * 1e-3), 1),
                               GBps=round(byt / (ms[mode] * 1e-3) / 1e9, 1),
                               hbm_frac=round(byt / (ms[mode] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                               alg_bytes_per_call=int(byt), snapshots=snap, state_update=upd)
            log("multi-token decode (%s): %.1f us/call, %.0f GB/s"
                % (mode, ms[mode] * 1e3, multi[mode]["GBps"]))
    lowp = None
    if not args.no_decode:
        wd = gen.WORKLOADS[4]
        ms = run_decode_lowp(wd, 30, 5)
        lowp = {"workload": wd.name}
        for name, v in ms.items():
            byt = lowp_bytes(wd, "int16" if name == "int16" else "f16")
            lowp[name] = dict(us_per_step=round(v * 1e3, 2),
                              GBps=round(byt / (v * 1e-3) / 1e9, 1),
                              hbm_frac=round(byt / (v * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                              alg_bytes_per_step=int(byt))
            log("decode, %s state: %.1f us/step, %.0f GB/s" % (name, v * 1e3, lowp[name]["GBps"]))
    bwd = None
    if not args.no_decode:
        bms = run_backward(w, 10, 10)
        bb = bwd_bytes(w, io_bytes)
        bwd = dict(us_per_call=round(bms * 1e3, 2), tokens_per_s=round(tokens / (bms * 1e-3), 1),
                   over_forward=round(bms / step_ms, 3),
                   must_move_bytes=int(bb), GBps=round(bb / (bms * 1e-3) / 1e9, 1),
                   hbm_frac=round(bb / (bms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                   gradients="dx, ddt, dA, dB, dC, dD, dinit (fp32)")
        log("backward: %.1f us/call (%.2fx the forward)" % (bms * 1e3, bms / step_ms))
    layer = None
    if not args.no_decode:
        wd = gen.WORKLOADS[4]
        fms, dms_ = run_layer_interface(w, wd, args.steps, args.warmup)
        zb = w.batch * w.seqlen * w.nheads * w.headdim * io_bytes
        layer = dict(options="dt_bias + softplus + z gate",
                     forward_us=round(fms * 1e3, 2), forward_tokens_per_s=round(tokens / (fms * 1e-3), 1),
                     forward_over_plain=round(fms / step_ms, 4), z_bytes=int(zb),
                     decode_workload=wd.name, decode_us_per_step=round(dms_ * 1e3, 2),
                     decode_over_plain=(round(dms_ / med, 4) if decode else None))
        log("layer interface: forward %.1f us (%.3fx plain), decode %.1f us/step"
            % (fms * 1e3, fms / step_ms, dms_ * 1e3))
    copy_gbps = run_copy_reference()
    log("device copy reference: %.0f GB/s" % copy_gbps)

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        cpu = run_cpu_baseline(w)
        log("oracle: %.3e tokens/s on %d threads" % (cpu["value"], cpu["cores"]))

    try:
        sha = subprocess.run(["git", "rev-parse", "--short", "HEAD"], cwd=ROOT,
                             capture_output=True, text=True).stdout.strip() or None
    except Exception:
        sha = None

    rec = {
        "metric": "SSD forward tokens/sec at 2.7B-layer shape + % bf16 MFMA roofline; decode GB/s",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "nheads": w.nheads,
                   "headdim": w.headdim, "dstate": w.dstate, "ngroups": w.ngroups,
                   "chunk_size": w.chunk_size, "io_dtype": w.io_dtype,
                   "init_state": w.init_state, "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "median_ms_per_step": round(fw["median_ms"], 4),
        "min_ms_per_step": round(fw["min_ms"], 4),
        "settle_ms": fw["settle_ms"],
        "settle_calls": fw["settle_calls"],
        "state_path": PATH_NAMES[fw["path"]],
        "forward_bf16_mfma_frac": round(fwd_flops / (step_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        "chunk_kernels_bf16_mfma_frac": round(chunk_flops / (chunk_ms * 1e-3) / 1e12
                                              / BF16_PEAK_TFLOPS, 4),
        "kernels": kernels,
        "forward_y_io_dtype": y_io,
        "configs": configs,
        "decode": decode,
        "backward": bwd,
        "decode_multi": multi,
        "decode_lowp_state": lowp,
        "layer_interface": layer,
        "hbm_copy_reference_GBps": round(copy_gbps, 1),
        "wall_s_timed": round(wall, 4),
        "git": sha,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
