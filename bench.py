#!/usr/bin/env python3
"""Throughput of one MI355X's share of an MoE layer (expert parallelism).

A step is one pass of the whole share over one batch of tokens: router
logits, top-k and combine weights; dispatch (rows grouped by local expert);
the local experts' SwiGLU MLPs as two grouped GEMMs; combine (weighted top-k
sum in token order). Default workload: a DeepSeek-R1-shaped layer, rank 0 of
EP = 8 (T = 16384 tokens, H = 7168, I = 2048, 256 experts of which 32 are
local, top-8), seeded synthetic inputs resident in HBM before timing.

Prints ONE JSON line on stdout; everything else goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s on 1 GPU; grouped-GEMM % MFMA peak; dispatch/combine % HBM"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E peak
STAGES = ["route", "dispatch", "gemm1_gate_up_swiglu", "gemm2_down", "combine"]
# GEMM1 HBM traffic comes from rocprofv3 counter runs summarised (by
# --summarize-counters) in this file; it is reported only while the kernel
# sources still hash to what was profiled.
COUNTERS_MD = os.path.join(ROOT, "profiles", "counters_dsr1_ep8_share.md")
GEMM1_SOURCES = ["expert_token_routing_amd/csrc/expert_ffn.hip", "expert_token_routing_amd/csrc/gemm_dma.h",
                 "expert_token_routing_amd/csrc/gemm_tile.h", "expert_token_routing_amd/csrc/moe_device.h"]
GEMM1_KERNEL = "moe::panel_gemm_kernel<true, false, false>"
CALIB_LIB = os.path.join(ROOT, "expert_token_routing_amd", "libmoe_calib.so")
COPY_KERNEL = "__amd_rocclr_copyBuffer"
DMA_CALIB_KERNEL = "(anonymous namespace)::dma_read_kernel"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    import workloads as W
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dsr1_ep8_share", choices=list(W.CONFIGS))
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle timing")
    ap.add_argument("--cpu-sample-tokens", type=int, default=16384,
                    help="tokens of the workload the CPU oracle runs on (bounded sample)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before timing, copy a buffer of this many MiB device to device once and read it once "
                         "more with the GEMMs' direct-to-LDS loads (libmoe_calib.so): reads and writes of known "
                         "size that scale hardware byte counters; 0 = off")
    ap.add_argument("--library-reference", action="store_true",
                    help="instead of the share, time torch.matmul / torch.bmm (hipBLASLt, bf16) on dense and batched "
                         "products of the workload's GEMM shapes and print one JSON line")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="print a markdown per-kernel summary of rocprofv3 --pmc output folders (one per counter "
                         "pass) and exit; see --profile-command")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print a markdown table of a rocprofv3 --kernel-trace --stats output folder and exit")
    ap.add_argument("--profile-command", default="",
                    help="with --summarize-*: the command(s) that produced the folders, quoted in the summary")
    ap.add_argument("--profile-title", default="", help="with --summarize-*: the summary's title")
    ap.add_argument("--cold-steps", type=int, default=5,
                    help="extra steps timed with a 1 GiB write between them (evicts L2 / Infinity Cache); 0 = off")
    ap.add_argument("--ep-sweep", default="",
                    help="comma-separated EP degrees (e.g. 1,2,4,8,16,32,64): instead of the single share, time "
                         "every rank's share of the workload's whole layer (e0 = r * E/ep) at each degree and "
                         "print one JSON line with the layer time per degree (max over ranks)")
    return ap.parse_args()


def gemm1_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for rel in GEMM1_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_gemm1_traffic():
    """(bytes per GEMM1 launch, note) from the committed counter summary, or
    (None, reason) when it is missing or the kernel changed since."""
    try:
        with open(COUNTERS_MD) as f:
            kv = dict(line.strip()[2:].split(": ", 1) for line in f if line.startswith("- ") and ": " in line)
    except OSError:
        return None, "no counter summary"
    if kv.get("gemm1_source_sha256") != gemm1_sources_sha256():
        return None, "kernel sources changed since the counters were taken"
    return (float(kv["gemm1_traffic_bytes_per_launch"]),
            f"rocprofv3 FETCH_SIZE/WRITE_SIZE, {os.path.relpath(COUNTERS_MD, ROOT)}")


def short_kernel_name(name):
    """Kernel name without its argument list (and without a leading 'void ')."""
    name = name.strip()
    if name.startswith("void "):
        name = name[5:]
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0 and i > 0:
            name = name[:i]
            break
    if len(name) > 72 and "<" in name:  # library kernels with long template arguments
        name = name[:name.index("<")] + "<...>"
    return name


def read_counter_dirs(dirs):
    """Per kernel: per-dispatch durations (ns) and per-dispatch counter
    values (summed over the rows a dispatch has), from rocprofv3 --pmc csv
    folders -- one folder per counter pass."""
    import csv
    import glob
    per = {}
    for d in dirs:
        for fn in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            with open(fn) as f:
                for r in csv.DictReader(f):
                    key = (fn, int(r["Dispatch_Id"]))
                    rec = per.setdefault(key, {"kernel": short_kernel_name(r["Kernel_Name"]),
                                               "dur": int(r["End_Timestamp"]) - int(r["Start_Timestamp"]), "c": {}})
                    rec["c"][r["Counter_Name"]] = rec["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    kern = {}
    for rec in per.values():
        k = kern.setdefault(rec["kernel"], {"dur": [], "c": {}})
        k["dur"].append(rec["dur"])
        for c, v in rec["c"].items():
            k["c"].setdefault(c, []).append(v)
    return kern


def summarize_counters(dirs, command, title):
    """Markdown per-kernel summary of rocprofv3 --pmc runs of a bench.py run
    with --copy-calibration-mib M (the copy and the direct-to-LDS read of M
    MiB are the byte-counter calibration). Derived figures, per dispatch:
    engine clock = GRBM_GUI_ACTIVE / 8 XCDs / duration; MFMA busy =
    SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / (GRBM_GUI_ACTIVE / 8);
    LDS bank-conflict share = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE;
    HBM bytes = FETCH_SIZE, WRITE_SIZE (KiB) x the calibration scale; read
    bytes by request size = 32 / 64 / 128 x TCC_EA0_RDREQ_{32B,64B,128B}_sum;
    L2 hit rate = TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum)."""
    import re

    import numpy as np
    kern = read_counter_dirs(dirs)
    m = re.search(r"--copy-calibration-mib (\d+)", command)
    known = int(m.group(1)) << 20 if m else None  # no calibration: no byte scales

    def mean(k, c):
        v = kern.get(k, {}).get("c", {}).get(c)
        return float(np.mean(v)) if v else None

    def calib(k, c):  # the largest dispatch of a calibration kernel: the M MiB one
        v = kern.get(k, {}).get("c", {}).get(c)
        return max(v) if v else None

    copy_f, copy_w = calib(COPY_KERNEL, "FETCH_SIZE"), calib(COPY_KERNEL, "WRITE_SIZE")
    dma_f = calib(DMA_CALIB_KERNEL, "FETCH_SIZE")
    f_scale = known / (copy_f * 1024.0) if (copy_f and known) else None
    w_scale = known / (copy_w * 1024.0) if (copy_w and known) else None
    dma_scale = known / (dma_f * 1024.0) if (dma_f and known) else None
    lines = [f"# {title}" if title else "# Counter summary", "",
             "rocprofv3 counter passes (one `--pmc` set per run) of the command(s) below, averaged per dispatch "
             "of each kernel.", "", "```", command, "```", ""]
    if known:
        lines += ["## Byte-counter calibration", "",
                  f"Known sizes: the device-to-device copy reads and writes {known >> 20} MiB "
                  f"(`{COPY_KERNEL}`); `{DMA_CALIB_KERNEL}` (libmoe_calib.so) reads the same {known >> 20} MiB once "
                  "with the 16-byte `buffer_load_dwordx4 ... lds` loads the GEMM operand stages use.", "",
                  "| calibration | counter | reads (KiB) | known (KiB) | scale |", "|---|---|---:|---:|---:|"]
        for name, c, v, sc in ((COPY_KERNEL, "FETCH_SIZE", copy_f, f_scale),
                               (COPY_KERNEL, "WRITE_SIZE", copy_w, w_scale),
                               (DMA_CALIB_KERNEL, "FETCH_SIZE", dma_f, dma_scale)):
            if v:
                lines.append(f"| `{name}` | {c} | {v:.0f} | {known / 1024:.0f} | {sc:.4f} |")
    req = [(COPY_KERNEL, "copy"), (DMA_CALIB_KERNEL, "direct-to-LDS read")]
    if known and any(calib(k, "TCC_EA0_RDREQ_sum") for k, _ in req):
        lines += ["", "Read requests the L2 sent to memory, by size (the same calibration dispatches):", "",
                  "| calibration | requests | 32 B | 64 B | 128 B | bytes by size / known |",
                  "|---|---:|---:|---:|---:|---:|"]
        for k, lab in req:
            tot = calib(k, "TCC_EA0_RDREQ_sum")
            if not tot:
                continue
            r32, r64, r128 = (calib(k, f"TCC_EA0_RDREQ_{b}_sum") or 0.0 for b in ("32B", "64B", "128B"))
            lines.append(f"| {lab} | {tot:.0f} | {r32:.0f} | {r64:.0f} | {r128:.0f} | "
                         f"{(32 * r32 + 64 * r64 + 128 * r128) / known:.4f} |")
    lines += ["", "## Per kernel", "",
              "| kernel | dispatches | avg (us) | clock (GHz) | MFMA busy | LDS conflict | HBM read (MB) | "
              "HBM write (MB) | HBM GB/s | read by req. size (MB) | L2 hit |",
              "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    kv = []
    order = sorted(kern, key=lambda k: -float(np.mean(kern[k]["dur"])) * len(kern[k]["dur"]))
    for k in order:
        if k in (COPY_KERNEL, DMA_CALIB_KERNEL):
            continue
        dur = float(np.mean(kern[k]["dur"]))
        n = min(len(v) for v in kern[k]["c"].values())  # counters taken in one pass only
        grbm, mf = mean(k, "GRBM_GUI_ACTIVE"), mean(k, "SQ_VALU_MFMA_BUSY_CYCLES")
        conf, lact = mean(k, "SQ_LDS_BANK_CONFLICT"), mean(k, "SQ_LDS_IDX_ACTIVE")
        fe, wr = mean(k, "FETCH_SIZE"), mean(k, "WRITE_SIZE")
        hit, miss = mean(k, "TCC_HIT_sum"), mean(k, "TCC_MISS_sum")
        rq = [mean(k, f"TCC_EA0_RDREQ_{b}_sum") for b in ("32B", "64B", "128B")]
        clk = grbm / 8 / dur if (grbm and dur > 20e3) else None  # short launches: fixed overhead dominates
        busy = mf / 1024 / (grbm / 8) if (mf is not None and grbm) else None
        rd = fe * 1024 * f_scale if (fe is not None and f_scale) else None
        wb = wr * 1024 * w_scale if (wr is not None and w_scale) else None
        gbs = (rd + wb) / dur if (rd is not None and wb is not None) else None
        by_size = (32 * (rq[0] or 0) + 64 * (rq[1] or 0) + 128 * (rq[2] or 0)) if any(
            v is not None for v in rq) else None

        def f(v, fmt):
            return "-" if v is None else format(v, fmt)
        lines.append(f"| `{k}` | {n} | {dur / 1e3:.1f} | {f(clk, '.2f')} | {f(busy and 100 * busy, '.1f')}"
                     f"{'%' if busy is not None else ''} | "
                     f"{f(conf / lact * 100 if (conf is not None and lact) else None, '.2f')}"
                     f"{'%' if (conf is not None and lact) else ''} | {f(rd and rd / 1e6, '.1f')} | "
                     f"{f(wb and wb / 1e6, '.1f')} | {f(gbs, '.0f')} | {f(by_size and by_size / 1e6, '.1f')} | "
                     f"{f(hit / (hit + miss) * 100 if (hit is not None and miss is not None and hit + miss > 0) else None, '.1f')}"
                     f"{'%' if (hit is not None and miss) else ''} |")
        if k == GEMM1_KERNEL and rd is not None and wb is not None:
            kv += [f"- gemm1_traffic_bytes_per_launch: {rd + wb:.0f}",
                   f"- gemm1_source_sha256: {gemm1_sources_sha256()}"]
    lines += ["", "HBM bytes use the copy's scales (read and write). MFMA busy and clock need GRBM_GUI_ACTIVE and "
              "SQ_VALU_MFMA_BUSY_CYCLES in the same pass; a '-' is a counter not collected.", ""]
    # the load path of the kernels that move most data, when its counters were taken
    mem = [k for k in order if mean(k, "TD_TD_BUSY_sum") is not None and mean(k, "TCP_TCC_READ_REQ_sum")
           and float(np.mean(kern[k]["dur"])) > 20e3 and k not in (COPY_KERNEL,)]
    if mem:
        lines += ["## Load path", "",
                  "Per dispatch; busy and stall shares are of the dispatch's cycles on each of the 256 CUs "
                  "(counter sum / 256 / (GRBM_GUI_ACTIVE / 8)). L2 latency = TCP_TCC_READ_REQ_LATENCY_sum / "
                  "TCP_TCC_READ_REQ_sum (cycles per L1-to-L2 read request); lines in flight per CU = requests x "
                  "latency / 256 / cycles (Little's law).", "",
                  "| kernel | L1->L2 reads | L2 hit | L2 latency (cyc) | lines in flight / CU | TA busy | "
                  "TD busy | TD waiting on L1 | L1 waiting on L2 |",
                  "|---|---:|---:|---:|---:|---:|---:|---:|---:|"]
        for k in mem:
            grbm = mean(k, "GRBM_GUI_ACTIVE")
            cyc = grbm / 8 if grbm else None
            req, lat = mean(k, "TCP_TCC_READ_REQ_sum"), mean(k, "TCP_TCC_READ_REQ_LATENCY_sum")
            hit, miss = mean(k, "TCC_HIT_sum"), mean(k, "TCC_MISS_sum")

            def share(c):
                v = mean(k, c)
                return "-" if (v is None or not cyc) else f"{100 * v / 256 / cyc:.0f}%"
            lat_c = lat / req if (lat and req) else None
            fl = req * lat_c / 256 / cyc if (lat_c and cyc) else None
            lines.append(f"| `{k}` | {req:.3g} | "
                         f"{'-' if hit is None or miss is None else f'{100 * hit / (hit + miss):.0f}%'} | "
                         f"{'-' if lat_c is None else f'{lat_c:.0f}'} | {'-' if fl is None else f'{fl:.0f}'} | "
                         f"{share('TA_TA_BUSY_sum')} | {share('TD_TD_BUSY_sum')} | {share('TD_TC_STALL_sum')} | "
                         f"{share('TCP_PENDING_STALL_CYCLES_sum')} |")
        lines.append("")
    if kv:
        lines += ["Recorded for bench.py's roofline (the gate/up GEMM's HBM bytes per launch and the hash of its "
                  "sources when they were taken):", ""] + kv
    return "\n".join(lines) + "\n"


def summarize_trace(d, command, title):
    """Markdown table of a rocprofv3 --kernel-trace --stats folder."""
    import csv
    import glob
    rows = []
    for fn in glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True):
        with open(fn) as f:
            rows += list(csv.DictReader(f))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    tot = sum(float(r["TotalDurationNs"]) for r in rows)
    lines = [f"# {title}" if title else "# Kernel trace", "", "```", command, "```", "",
             "| kernel | calls | avg (us) | min (us) | max (us) | share |", "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        lines.append(f"| `{short_kernel_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{100 * float(r['TotalDurationNs']) / tot:.1f}% |")
    return "\n".join(lines) + "\n"


def algorithmic(cfg, N, U, E_hit, fused_gather=True):
    """Algorithmic work of each stage for realised local rows N, source
    tokens with a local pick U and local experts with at least one row E_hit.
    In the fused forward, dispatch only builds the tables (GEMM1 reads the
    token rows in place); the row-moving dispatch of the standalone entry
    point is `dispatch_rows`. GEMM bytes: every weight of a used expert once,
    the input rows once, the output rows once."""
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    rows = dict(bytes=2.0 * U * H + 2.0 * N * H + 8.0 * T * k + 4.0 * N)
    return {
        "route": dict(flop=2.0 * T * E * H, bytes=2.0 * T * H + 4.0 * E * H + 4.0 * T * E + 8.0 * T * k),
        "dispatch": dict(bytes=8.0 * T * k + 4.0 * N) if fused_gather else rows,
        "gemm1_gate_up_swiglu": dict(flop=4.0 * N * H * I,
                                     bytes=4.0 * E_hit * H * I + 2.0 * (U if fused_gather else N) * H + 2.0 * N * I),
        "gemm2_down": dict(flop=2.0 * N * I * H, bytes=2.0 * E_hit * I * H + 2.0 * N * I + 2.0 * N * H),
        "combine": dict(bytes=2.0 * N * H + 2.0 * T * H + 8.0 * T * k),
        "dispatch_rows": rows,
    }


def calib_lib():
    """libmoe_calib.so (include/moe_calib.h), built beside libmoe.so."""
    import ctypes
    if not os.path.exists(CALIB_LIB):
        sys.exit(f"{CALIB_LIB} is missing: build with python -m expert_token_routing_amd.build_lib")
    cal = ctypes.CDLL(CALIB_LIB)
    cal.moe_calib_dma_read.restype = ctypes.c_int
    cal.moe_calib_dma_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    cal.moe_calib_mfma_loop.restype = ctypes.c_int
    cal.moe_calib_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double),
                                        ctypes.c_void_p]
    return cal


def mfma_attainable(stream, dev):
    """bf16 matrix-core rate of the register-only MFMA loop (no memory
    traffic), 2 and 1 waves per SIMD, best of 5 launches each (TFLOP/s)."""
    import ctypes

    import torch
    cal = calib_lib()
    sink = torch.zeros(1, dtype=torch.float32, device=dev)
    out = {}
    for wps, iters in ((2, 16000), (1, 32000)):
        flop = ctypes.c_double(0)
        best = None
        for _ in range(6):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            st = cal.moe_calib_mfma_loop(iters, wps, ctypes.c_void_p(sink.data_ptr()), ctypes.byref(flop),
                                         ctypes.c_void_p(stream.cuda_stream))
            e1.record(stream)
            if st != 0:
                sys.exit(f"moe_calib_mfma_loop failed with status {st}")
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            if best is None or ms < best:
                best = ms
        out[f"tflops_{wps}_waves_per_simd"] = round(flop.value / (best * 1e-3) / 1e12, 1)
    return out


def library_reference(args):
    """hipBLASLt (through torch.matmul / torch.bmm, bf16, float32 accumulate)
    on the workload's GEMM shapes: the dense products over all T tokens with
    one weight matrix, the batched products with E_local weight matrices of
    the mean rows per expert, and a square 8192 product. Context for what
    the vendor library reaches on this chip; nothing here is the share."""
    import numpy as np
    import torch

    import workloads as W
    cfg = W.CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    rows = (cfg.T * cfg.k * cfg.E_local) // cfg.E  # expected rows of the share
    per = max(1, rows // cfg.E_local)

    def rnd(*shape):
        return (torch.randn(*shape, device=dev, generator=g, dtype=torch.float32) * 0.05).to(torch.bfloat16)

    cases = [
        (f"dense [{cfg.T} x {cfg.H}] @ [{cfg.H} x {2 * cfg.I}]", lambda: (rnd(cfg.T, cfg.H), rnd(cfg.H, 2 * cfg.I)),
         torch.matmul, 2.0 * cfg.T * cfg.H * 2 * cfg.I),
        (f"dense [{cfg.T} x {cfg.I}] @ [{cfg.I} x {cfg.H}]", lambda: (rnd(cfg.T, cfg.I), rnd(cfg.I, cfg.H)),
         torch.matmul, 2.0 * cfg.T * cfg.I * cfg.H),
        (f"batched {cfg.E_local} x [{per} x {cfg.H}] @ [{cfg.H} x {2 * cfg.I}]",
         lambda: (rnd(cfg.E_local, per, cfg.H), rnd(cfg.E_local, cfg.H, 2 * cfg.I)), torch.bmm,
         2.0 * cfg.E_local * per * cfg.H * 2 * cfg.I),
        (f"batched {cfg.E_local} x [{per} x {cfg.I}] @ [{cfg.I} x {cfg.H}]",
         lambda: (rnd(cfg.E_local, per, cfg.I), rnd(cfg.E_local, cfg.I, cfg.H)), torch.bmm,
         2.0 * cfg.E_local * per * cfg.I * cfg.H),
        ("dense [8192 x 8192] @ [8192 x 8192]", lambda: (rnd(8192, 8192), rnd(8192, 8192)), torch.matmul,
         2.0 * 8192 ** 3),
    ]
    stream = torch.cuda.current_stream(dev)
    res = []
    for name, make, fn, flop in cases:
        a, b = make()  # both operands contiguous
        for _ in range(3):
            fn(a, b)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(11)]
        evs[0].record(stream)
        for i in range(10):
            fn(a, b)
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        ms = float(np.median([evs[i].elapsed_time(evs[i + 1]) for i in range(10)]))
        tf = flop / (ms * 1e-3) / 1e12
        res.append({"case": name, "us": round(ms * 1e3, 1), "tflops": round(tf, 1),
                    "frac_mfma_bf16": round(tf / PEAK_BF16_TFLOPS, 4)})
        log(f"[libref] {name}: {ms * 1e3:.1f} us, {tf:.0f} TFLOP/s")
        del a, b
    print(json.dumps({"metric": "vendor library (hipBLASLt via torch, bf16) on the workload's GEMM shapes",
                      "workload": cfg.name, "mfma_attainable": mfma_attainable(stream, dev), "cases": res,
                      "torch": torch.__version__}), flush=True)


def cpu_baseline(inp, sample_tokens):
    """The CPU oracle, as it stands, on the first `sample_tokens` tokens of the
    same workload (all of the rank's experts)."""
    import numpy as np
    import oracle.moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas = [d for d in threadpool_info() if d.get("user_api") == "blas"]
        cores = int(blas[0]["num_threads"]) if blas else len(os.sched_getaffinity(0))
        blas_name = blas[0].get("internal_api", "?") if blas else "?"
    except Exception:  # pragma: no cover
        cores, blas_name = len(os.sched_getaffinity(0)), "?"
    cfg = inp.cfg
    S = min(sample_tokens, cfg.T)
    x = inp.x[:S]
    # repeat the whole sample until about 10 s of CPU work have been timed
    runs = 0
    t0 = time.perf_counter()
    while True:
        O.oracle_forward(x, inp.w_router, inp.bias, inp.w_gate_up, inp.w_down, cfg.k, cfg.e0, cfg.E_local,
                         cfg.renormalize)
        runs += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or runs >= 20:
            break
    cpu = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": S * runs / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {S} of {cfg.T} tokens of {cfg.name}, all {cfg.E_local} local experts, "
                      f"float64 numpy ({blas_name}), {runs} runs in {dt:.1f} s on {cpu}"}


def ep_sweep(args):
    """Every rank's share of the workload's whole layer at each EP degree,
    run one after another on this GPU. Under expert parallelism the ranks run
    their shares side by side, so the layer time at degree ep (before the
    exchange of partial outputs) is the slowest rank's share time."""
    import dataclasses

    import numpy as np
    import torch

    import expert_token_routing_amd as M
    import workloads as W

    base = W.CONFIGS[args.workload]
    degrees = [int(v) for v in args.ep_sweep.split(",") if v.strip()]
    for ep in degrees:
        if ep < 1 or base.E % ep:
            sys.exit(f"--ep-sweep: EP degree {ep} does not divide E = {base.E}")
    cfg = dataclasses.replace(base, name=base.name + "_layer", e0=0, E_local=base.E)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[sweep] generating {cfg.name} inputs (all {cfg.E} experts)")
    inp = W.make_inputs(cfg)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    x = bf(inp.x)
    wr = torch.from_numpy(inp.w_router).to(dev)
    bias = None if inp.bias is None else torch.from_numpy(inp.bias).to(dev)
    gu = bf(inp.w_gate_up)
    dn = bf(inp.w_down)
    del inp
    y = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps + 1)]
    for row in evs:
        for ev in row:
            ev.record(stream)  # creates the underlying HIP event
    rows = []
    for ep in degrees:
        El = cfg.E // ep
        ws = torch.empty(M.forward_workspace_size(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, El), dtype=torch.uint8,
                         device=dev)
        lay = M.forward_workspace_layout(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, El)
        share_ms, stage_ms, n_rows = [], [], []
        log(f"[sweep] ep={ep} E_local={El}: {ep} shares")
        for r in range(ep):
            gu_r, dn_r = gu[r * El:(r + 1) * El], dn[r * El:(r + 1) * El]
            for _ in range(args.warmup):
                M.moe_forward_profiled(x, wr, bias, gu_r, dn_r, cfg.k, r * El, cfg.renormalize, y, ws, evs[0],
                                       stream=stream)
            for i in range(args.steps):
                M.moe_forward_profiled(x, wr, bias, gu_r, dn_r, cfg.k, r * El, cfg.renormalize, y, ws,
                                       evs[i + 1], stream=stream)
            torch.cuda.synchronize()
            st = np.array([[evs[i + 1][j].elapsed_time(evs[i + 1][j + 1]) for j in range(5)]
                           for i in range(args.steps)]).mean(0)
            stage_ms.append(st)
            share_ms.append(float(st.sum()))
            n_rows.append(int(ws[lay["offsets"] + 4 * El:lay["offsets"] + 4 * El + 4].view(torch.int32).item()))
        share_ms = np.array(share_ms)
        stage_ms = np.array(stage_ms)
        n_rows = np.array(n_rows)
        gemm_ms = stage_ms[:, 2] + stage_ms[:, 3]
        gemm_tf = 6.0 * n_rows * cfg.H * cfg.I / (gemm_ms * 1e-3) / 1e12
        worst = int(share_ms.argmax())
        rows.append({
            "ep": ep, "E_local": El,
            "layer_ms": round(float(share_ms.max()), 4),
            "layer_tokens_per_s": round(cfg.T / (share_ms.max() * 1e-3), 1),
            "share_ms_mean": round(float(share_ms.mean()), 4),
            "imbalance_max_over_mean": round(float(share_ms.max() / share_ms.mean()), 4),
            "rows_per_rank_max": int(n_rows.max()), "rows_per_rank_mean": round(float(n_rows.mean()), 1),
            "grouped_gemm_tflops_mean": round(float(gemm_tf.mean()), 2),
            "grouped_gemm_frac_mfma_bf16_mean": round(float(gemm_tf.mean()) / PEAK_BF16_TFLOPS, 4),
            "slowest_rank": worst,
            "slowest_rank_stage_us": {n: round(float(v) * 1e3, 2) for n, v in zip(STAGES, stage_ms[worst])},
        })
        log(f"[sweep] ep={ep}: layer {share_ms.max():.3f} ms (mean share {share_ms.mean():.3f} ms), "
            f"GEMM {gemm_tf.mean():.0f} TFLOP/s")
        del ws
    print(json.dumps({
        "metric": "EP-share sweep: layer time at each EP degree = slowest rank's share (partial-output exchange "
                  "not included), every share run on this one GPU",
        "workload": cfg.name, "T": cfg.T, "H": cfg.H, "I": cfg.I, "E": cfg.E, "k": cfg.k,
        "renormalize": cfg.renormalize, "steps_per_share": args.steps, "warmup_per_share": args.warmup,
        "dtype": "bf16", "data": "synthetic (seeded numpy PCG64, shapes of the named workload; no trained weights)",
        "rows": rows,
    }), flush=True)


def main():
    args = parse()
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters, args.profile_command, args.profile_title), end="")
        return
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.profile_command, args.profile_title), end="")
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU's share of the MoE layer; runs on more than one GPU are not part "
              "of this build (--gpus must be 1)", file=sys.stderr)
        sys.exit(2)
    if args.ep_sweep:
        ep_sweep(args)
        return
    if args.library_reference:
        library_reference(args)
        return

    import numpy as np
    import torch

    import expert_token_routing_amd as M
    import workloads as W

    cfg = W.CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] generating {cfg.name} inputs")
    inp = W.make_inputs(cfg)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    x = bf(inp.x)
    wr = torch.from_numpy(inp.w_router).to(dev)
    bias = None if inp.bias is None else torch.from_numpy(inp.bias).to(dev)
    gu = bf(inp.w_gate_up)
    dn = bf(inp.w_down)
    y = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(M.forward_workspace_size(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.E_local),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def new_events(n):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(n)]
        for row in evs:
            for ev in row:
                ev.record(stream)  # creates the underlying HIP event
        return evs

    def step(evs):
        M.moe_forward_profiled(x, wr, bias, gu, dn, cfg.k, cfg.e0, cfg.renormalize, y, ws, evs, stream=stream)

    if args.copy_calibration_mib > 0:
        nb = args.copy_calibration_mib << 20
        src = torch.full((nb,), 7, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: {nb} bytes read, {nb} bytes written")
        import ctypes
        cal = calib_lib()
        st = cal.moe_calib_dma_read(ctypes.c_void_p(src.data_ptr()), nb, ctypes.c_void_p(stream.cuda_stream))
        if st != 0:
            sys.exit(f"moe_calib_dma_read failed with status {st}")
        torch.cuda.synchronize()
        log(f"[bench] direct-to-LDS read calibration: {nb} bytes read")
        del src, dst

    log(f"[bench] warmup {args.warmup}")
    wev = new_events(1)
    for _ in range(args.warmup):
        step(wev[0])
    torch.cuda.synchronize()

    # the timed steps: plain moe_forward calls (the entry point a caller uses)
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        M.moe_forward(x, wr, bias, gu, dn, cfg.k, cfg.e0, cfg.renormalize, y=y, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the same number of steps again through moe_forward_profiled, whose
    # events on the compute stream give each stage's device time
    evs = new_events(args.steps)
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    stage_ms = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(5)] for i in range(args.steps)])
    stage_avg = stage_ms.mean(0)
    step_ev = stage_ms.sum(1)  # per-step device time between the first and last event
    log("[bench] stage ms: " + ", ".join(f"{n}={v:.3f}" for n, v in zip(STAGES, stage_avg)))

    cold = None
    if args.cold_steps > 0:
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        cev = new_events(args.cold_steps)
        torch.cuda.synchronize()
        for i in range(args.cold_steps):
            scratch.fill_(i & 0xFF)
            step(cev[i])
        torch.cuda.synchronize()
        cms = np.array([[cev[i][j].elapsed_time(cev[i][j + 1]) for j in range(5)] for i in range(args.cold_steps)])
        cold = {"ms_per_step": float(cms.sum(1).mean()),
                "stage_ms": {n: round(float(v), 4) for n, v in zip(STAGES, cms.mean(0))}}
        del scratch

    # moe_forward_fused: the combine of single-selection tokens in the down
    # GEMM's epilogue, timed the same way right after (same inputs, same y)
    fev = new_events(args.steps)
    for _ in range(max(2, args.warmup // 4)):
        M.moe_forward_profiled(x, wr, bias, gu, dn, cfg.k, cfg.e0, cfg.renormalize, y, ws, wev[0], stream=stream,
                               fused=True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(args.steps):
        M.moe_forward_fused(x, wr, bias, gu, dn, cfg.k, cfg.e0, cfg.renormalize, y=y, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    fused_wall = time.perf_counter() - t1
    for i in range(args.steps):
        M.moe_forward_profiled(x, wr, bias, gu, dn, cfg.k, cfg.e0, cfg.renormalize, y, ws, fev[i], stream=stream,
                               fused=True)
    torch.cuda.synchronize()
    fused_stage = np.array([[fev[i][j].elapsed_time(fev[i][j + 1]) for j in range(5)]
                            for i in range(args.steps)]).mean(0)
    log("[bench] fused-combine stage ms: " + ", ".join(f"{n}={v:.3f}" for n, v in zip(STAGES, fused_stage)))

    # realised routing of the timed steps (identical every step)
    lay = M.forward_workspace_layout(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.E_local)
    offs = ws[lay["offsets"]:lay["offsets"] + 4 * (cfg.E_local + 1)].view(torch.int32).cpu().numpy()
    inv = ws[lay["inv"]:lay["inv"] + 4 * cfg.T * cfg.k].view(torch.int32).reshape(cfg.T, cfg.k).cpu().numpy()
    N = int(offs[-1])
    U = int((inv >= 0).any(1).sum())
    single = int(((inv >= 0).sum(1) == 1).sum())
    fused = cfg.H % 32 == 0 and cfg.T * cfg.H * 2 < 2 ** 31
    E_hit = int((np.diff(offs) > 0).sum())
    work = algorithmic(cfg, N, U, E_hit, fused)

    # the standalone dispatch entry point (tables + rows moved into x_perm),
    # timed on its own with the forward's top-k ids
    idx = ws[lay["topk_idx"]:lay["topk_idx"] + 4 * cfg.T * cfg.k].view(torch.int32).reshape(cfg.T, cfg.k)
    cap = cfg.capacity
    d_out = dict(counts=torch.empty(cfg.E, dtype=torch.int32, device=dev),
                 offsets=torch.empty(cfg.E_local + 1, dtype=torch.int32, device=dev),
                 perm_src=torch.empty(cap, dtype=torch.int32, device=dev),
                 inv=torch.empty(cfg.T * cfg.k, dtype=torch.int32, device=dev),
                 x_perm=torch.empty((cap, cfg.H), dtype=torch.bfloat16, device=dev))
    d_ws = torch.empty(M.lib().moe_dispatch_workspace_size(cfg.T, cfg.E, cfg.k), dtype=torch.uint8, device=dev)
    for _ in range(2):
        M.moe_dispatch(x, idx, cfg.E, cfg.e0, cfg.E_local, workspace=d_ws, **d_out)
    nd = max(5, args.steps // 2)
    dev_ev = [torch.cuda.Event(enable_timing=True) for _ in range(nd + 1)]
    dev_ev[0].record(stream)
    for i in range(nd):
        M.moe_dispatch(x, idx, cfg.E, cfg.e0, cfg.E_local, workspace=d_ws, **d_out)
        dev_ev[i + 1].record(stream)
    torch.cuda.synchronize()
    d_ms = float(np.mean([dev_ev[i].elapsed_time(dev_ev[i + 1]) for i in range(nd)]))
    del d_out, d_ws

    # the combine alone, bf16 output and float32 partial output, on the
    # forward's own expert outputs, selections and weights
    n_out = max(N, 1)
    c_out = ws[lay["expert_out"]:lay["expert_out"] + 2 * n_out * cfg.H].view(torch.bfloat16).view(n_out, cfg.H)
    c_inv = ws[lay["inv"]:lay["inv"] + 4 * cfg.T * cfg.k].view(torch.int32)
    c_w = ws[lay["topk_w"]:lay["topk_w"] + 4 * cfg.T * cfg.k].view(torch.float32).view(cfg.T, cfg.k)
    y32 = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device=dev)
    y16 = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev)
    comb_ms = {}
    for name, fn, yy in (("bf16", M.moe_combine, y16), ("f32", M.moe_combine_f32, y32)) * 2:
        fn(c_out, c_inv, c_w, y=yy)
        c_ev = [torch.cuda.Event(enable_timing=True) for _ in range(nd + 1)]
        c_ev[0].record(stream)
        for i in range(nd):
            fn(c_out, c_inv, c_w, y=yy)
            c_ev[i + 1].record(stream)
        torch.cuda.synchronize()
        comb_ms[name] = float(np.mean([c_ev[i].elapsed_time(c_ev[i + 1]) for i in range(nd)]))
    f32_bytes = work["combine"]["bytes"] + 2.0 * cfg.T * cfg.H
    f32_gbs = f32_bytes / (comb_ms["f32"] * 1e-3) / 1e9
    combine_f32 = {"us": round(comb_ms["f32"] * 1e3, 2), "gbs": round(f32_gbs, 1),
                   "frac_hbm": round(f32_gbs / PEAK_HBM_GBS, 4), "bf16_us": round(comb_ms["bf16"] * 1e3, 2),
                   "note": "moe_combine_f32 (float32 partial output) and moe_combine, each timed alone on the "
                           "forward's expert outputs"}
    del y32, y16

    stages = {}
    for n, ms in zip(STAGES, stage_avg):
        s = {"us": round(float(ms) * 1e3, 2)}
        if "flop" in work[n]:
            s["tflops"] = round(work[n]["flop"] / (ms * 1e-3) / 1e12, 2)
        if "bytes" in work[n]:
            s["gbs"] = round(work[n]["bytes"] / (ms * 1e-3) / 1e9, 1)
        if n.startswith("gemm"):
            s["frac_mfma_bf16"] = round(s["tflops"] / PEAK_BF16_TFLOPS, 4)
            s["frac_hbm"] = round(s["gbs"] / PEAK_HBM_GBS, 4)
        if n in ("dispatch", "combine"):
            s["frac_hbm"] = round(s["gbs"] / PEAK_HBM_GBS, 4)
        stages[n] = s
    if fused:
        stages["dispatch"]["note"] = "tables only; GEMM1 gathers the token rows in place"
    d_gbs = work["dispatch_rows"]["bytes"] / (d_ms * 1e-3) / 1e9
    dispatch_rows = {"us": round(d_ms * 1e3, 2), "gbs": round(d_gbs, 1), "frac_hbm": round(d_gbs / PEAK_HBM_GBS, 4),
                     "note": "moe_dispatch entry point (tables + token rows copied to x_perm), timed alone"}

    # GEMM1's bound from its arithmetic intensity: flop per algorithmic byte
    # against the ridge point of the bf16 matrix peak and the HBM peak
    w1 = work["gemm1_gate_up_swiglu"]
    intensity = w1["flop"] / w1["bytes"]
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    g1 = w1["flop"] / (stage_avg[2] * 1e-3) / 1e12
    g1_gbs = w1["bytes"] / (stage_avg[2] * 1e-3) / 1e9
    traffic, traffic_note = recorded_gemm1_traffic() if cfg.name == "dsr1_ep8_share" else (None, "other workload")
    if intensity >= ridge:
        roofline = {"bound": "mfma", "kernel": "grouped GEMM1 (gate/up + SwiGLU)",
                    "achieved": round(g1, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(g1 / PEAK_BF16_TFLOPS, 4)}
    else:
        roofline = {"bound": "hbm", "kernel": "grouped GEMM1 (gate/up + SwiGLU)",
                    "achieved": round(g1_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(g1_gbs / PEAK_HBM_GBS, 4)}
    # the matrix-core rate this chip sustains (register-only MFMA loop), as
    # context for the spec peak the fractions use
    attain = mfma_attainable(stream, dev)
    att = attain["tflops_2_waves_per_simd"]
    log(f"[bench] register-only MFMA loop: {attain}")
    roofline.update({"traffic": traffic, "traffic_unit": "HBM bytes per launch", "traffic_source": traffic_note,
                     "intensity_flop_per_byte": round(intensity, 1), "ridge_flop_per_byte": round(ridge, 1),
                     "algorithmic_bytes": w1["bytes"], "algorithmic_flop": w1["flop"],
                     "attainable_peak": att, "frac_of_attainable": round(g1 / att, 4)})
    # the router: logits as three bf16 products (the float32 weight split into
    # three bf16 planes, exact), so 3 x 2 T E H matrix-core flop, then top-k
    # over the float32 logits (and the partial sums of a split k range)
    r_flop = 3 * 2.0 * cfg.T * cfg.E * cfg.H
    r_us = float(stage_avg[0]) * 1e3
    r_tf = r_flop / (r_us * 1e-6) / 1e12
    # top-k reads the logits and one partial sum and writes the logits back
    # (12 T E bytes) and the selection (8 T k); the split reads the float32
    # weight and writes three bf16 planes (10 E H). The logits kernel's own
    # loads and stores overlap its matrix work.
    topk_bytes = 12.0 * cfg.T * cfg.E + 8.0 * cfg.T * cfg.k
    split_bytes = 10.0 * cfg.E * cfg.H
    floor_us = (r_flop / (att * 1e12) + (topk_bytes + split_bytes) / (PEAK_HBM_GBS * 1e9)) * 1e6
    route_roofline = {"bound": "mfma", "kernel": "route: bf16x3 split logits, then top-k",
                      "mfma_flop": r_flop, "achieved": round(r_tf, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                      "frac": round(r_tf / PEAK_BF16_TFLOPS, 4), "frac_of_attainable": round(r_tf / att, 4),
                      "floor_us": round(floor_us, 1),
                      "floor_note": "three bf16 products at the attainable MFMA rate, plus the split's and the "
                                    "top-k's bytes at the HBM peak"}
    gemm_ms = stage_avg[2] + stage_avg[3]
    gemm_tflops = 6.0 * N * cfg.H * cfg.I / (gemm_ms * 1e-3) / 1e12
    ms_per_step = wall / args.steps * 1e3
    total_flop = 6.0 * N * cfg.H * cfg.I + 2.0 * cfg.T * cfg.E * cfg.H
    result = {
        "metric": METRIC,
        "value": round(cfg.T * args.steps / wall, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded numpy PCG64, shapes of the named workload; no trained weights)",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "I": cfg.I, "E": cfg.E, "k": cfg.k,
                   "e0": cfg.e0, "E_local": cfg.E_local, "renormalize": cfg.renormalize,
                   "parallelism": "one EP rank's share on 1 GPU"},
        "roofline": roofline,
        "grouped_gemm": {"tflops": round(gemm_tflops, 2), "frac_mfma_bf16": round(gemm_tflops / PEAK_BF16_TFLOPS, 4),
                         "frac_of_attainable": round(gemm_tflops / att, 4)},
        "route_roofline": route_roofline,
        "mfma_attainable": dict(attain, note="register-only v_mfma_f32_16x16x32_bf16 loop, libmoe_calib.so"),
        "stages": stages,
        "dispatch_rows": dispatch_rows,
        "combine_f32": combine_f32,
        "fused_combine": {
            "value": round(cfg.T * args.steps / fused_wall, 1), "unit": "tokens/s",
            "ms_per_step": round(fused_wall / args.steps * 1e3, 4),
            "stage_us": {n: round(float(v) * 1e3, 2) for n, v in zip(STAGES, fused_stage)},
            "tokens_single_local_pick": single,
            "note": "moe_forward_fused: tokens with exactly one local selection are weighted and written to y by "
                    "the down GEMM's epilogue, the combine kernel sums the rest; y is bit-identical to "
                    "moe_forward's"},
        "layer_tflops": round(total_flop / (ms_per_step * 1e-3) / 1e12, 2),
        "step_ms_events": {"p10": round(float(np.percentile(step_ev, 10)), 4),
                           "p50": round(float(np.percentile(step_ev, 50)), 4),
                           "p90": round(float(np.percentile(step_ev, 90)), 4),
                           "note": "per-step device time from the stage events of the moe_forward_profiled pass"},
        "realised": {"N_local_rows": N, "U_tokens_with_local_pick": U,
                     "rows_per_local_expert_max": int(np.diff(offs).max()),
                     "local_experts_empty": int((np.diff(offs) == 0).sum())},
        "cold": cold,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle on {args.cpu_sample_tokens} tokens")
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_sample_tokens)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
