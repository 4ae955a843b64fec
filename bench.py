#!/usr/bin/env python3
"""Benchmark of the online-softmax attention hot path on one MI355X.

One step runs every operation of the path once on its standard workload,
inputs already resident in HBM:

  softmax   osm_softmax_rows        4096 x 32000 fp32, N(0,9) + one spike/row in [20,90)
                                    (rows held on chip between the passes: 8 B/elem)
  softmax_2pass osm_softmax_rows_twopass  the same input, every row read twice from memory
                                    (the pages' two-pass count: 12 B/elem)
  fwd       osm_attn_fwd            bf16 B=4 H=32 N=4096 d=128, non-causal   (the headline)
  fwd_causal osm_attn_fwd           bf16 B=8 H=16 N=8192 d=128, causal, lengths U[1024,8192]
  decode    osm_attn_decode_splitkv bf16 B=16 Hq=32 Hkv=8 d=128, L U[4096,32768], 256-key pieces
                                    (piece summaries + merge)
  merge_lse osm_merge_lse           8 normalized pieces of a 524288-row d=128 bf16 output
                                    (log-sum-exp merge of results over disjoint key sets)
  extend    osm_attn_extend         bf16 B=16 Hq=32 Hkv=8 d=128, 4096 new keys per call folded
                                    into a persisted (m, l, O~) state (streaming attention)
  fwd_fp8   osm_attn_fwd_fp8        the fwd workload with OCP E4M3 Q, K, V (both products on the FP8
                                    matrix instruction; peak 5033 TFLOP/s)
  bwd       osm_attn_bwd            backward of the fwd workload (dQ, dK, dV from O, LSE, dO)
  bwd_causal osm_attn_bwd           backward of the fwd_causal workload
  fwd_d64   osm_attn_fwd            bf16 B=4 H=64 N=4096 d=64, non-causal (the headline's flops
                                    and bytes at head dim 64)
  bwd_d64   osm_attn_bwd            backward of the fwd_d64 workload

Each call is timed with HIP events on the stream it runs on (torch's current
stream); ``value`` is the headline forward's TFLOP/s (mean over the timed
steps; the median and minimum are reported beside it).  The CPU oracle is
timed on a bounded sample of the headline workload as a reported baseline.
After the timed steps, two reference kernels (libosm_probe.so: a streaming
copy and a matrix-core loop) are timed once as "achievable" context.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME]
       python bench.py --sweep      (the forward over sequence lengths 1K-32K, head dims
                                     128 and 64, causal or not: one JSON line each)
       python bench.py --sweep --sweep-bwd   (the same for the backward)
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOP/s & % MFMA peak (N=4K/32K); softmax/decode GB/s & % HBM peak"
PEAK_BF16_TFLOPS = 256 * 2.4e9 * 4096 / 1e12     # 2516.6 dense bf16 MFMA
PEAK_FP8_TFLOPS = 256 * 2.4e9 * 8192 / 1e12      # 5033.2 dense fp8 MFMA
PEAK_HBM_GBS = 8000.0
PROFILE_FWD = os.path.join(ROOT, "profiles", "attn_fwd_bf16_d128_B4_H32_N4096.md")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def bf16_dev(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


KERNEL_SOURCES = {"fwd": "attn_fwd.hip", "fwd_causal": "attn_fwd.hip", "softmax": "softmax_rows.hip",
                  "softmax_2pass": "softmax_rows.hip",
                  "decode": "decode.hip", "merge_lse": "merge_lse.hip", "extend": "decode.hip",
                  "bwd": "attn_bwd.hip", "bwd_causal": "attn_bwd.hip", "fwd_fp8": "attn_fwd_fp8.hip",
                  "fwd_d64": "attn_fwd.hip", "bwd_d64": "attn_bwd.hip"}
WORKLOADS = ["softmax", "softmax_2pass", "fwd", "fwd_causal", "decode", "merge_lse", "extend", "bwd",
             "bwd_causal", "fwd_fp8", "fwd_d64", "bwd_d64"]


def source_hash(name):
    """sha256 (first 16 hex digits) of the kernel source a workload runs."""
    import hashlib
    path = os.path.join(ROOT, "exact_attention_online_softmax_amd", "csrc", KERNEL_SOURCES[name])
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profile(path, name):
    """HBM bytes per launch recorded by the rocprofv3 counter runs summarized
    in `path`, or None when absent or taken on a different kernel source."""
    vals = {}
    try:
        with open(path) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    vals[k.strip()] = v.strip()
    except OSError:
        return None
    if vals.get("kernel_source_sha256_16") != source_hash(name):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (or the platform string)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def achievable(torch):
    """Rates of two reference kernels on this GPU (libosm_probe.so), each the
    median of 20 launches, each timed with HIP events on its own: a streaming copy
    of 1 GiB (GB/s of bytes read + written) and a bf16 matrix-core loop on
    N(0, 1) operands (TFLOP/s) with one 256-thread workgroup per compute unit,
    i.e. one wave per SIMD, as the attention forward runs."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "exact_attention_online_softmax_amd", "libosm_probe.so"))
    vp = ctypes.c_void_p
    lib.osmprobe_copy.argtypes = [vp, vp, ctypes.c_size_t, vp]
    lib.osmprobe_mfma_bf16.argtypes = [vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    stream = vp(torch.cuda.current_stream().cuda_stream)
    cus = torch.cuda.get_device_properties(0).multi_processor_count

    def timed(fn, reps=20):
        # each launch timed on its own (the stream drained before it)
        fn()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts)) / 1e3

    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    t_copy = timed(lambda: lib.osmprobe_copy(vp(src.data_ptr()), vp(dst.data_ptr()), nbytes, stream))
    del src, dst
    res = {"copy_GBps": round(2 * nbytes / t_copy / 1e9, 1),
           "copy": "1 GiB streaming copy (nontemporal 16-byte buffer loads and stores, 32 KiB per workgroup), "
                   "bytes read + written"}
    g = np.random.default_rng(12345)
    grid, iters = cus, 4096
    ops = torch.from_numpy(g.standard_normal(grid * 512 * 128, dtype=np.float32)).to("cuda").to(torch.bfloat16)
    out = torch.empty(grid * 512, dtype=torch.float32, device="cuda")
    for threads in (256, 512):
        t = timed(lambda: lib.osmprobe_mfma_bf16(vp(ops.data_ptr()), vp(out.data_ptr()), grid, threads, iters,
                                                 stream))
        res[f"mfma_bf16_TFLOPs_{threads // 256}wave_per_simd"] = round(grid * threads // 64 * iters * 8 * 32768.0
                                                                       / t / 1e12, 1)
    res["mfma"] = (f"v_mfma_f32_32x32x16_bf16 chains (4 accumulators per wave) on N(0,1) operands, {grid} "
                   f"workgroups of 4 or 8 waves, no memory traffic in the loop")
    return res


def cpu_baseline(inp, seconds):
    """The oracle on the first rows of the headline workload, sized to take
    about `seconds` on the host's cores."""
    import oracle
    orc = oracle.load()
    q, k, v = inp.widened()
    B, H, N, d = q.shape
    flops_per_row = 4.0 * N * d
    n = 64
    t0 = time.perf_counter()
    orc.attention(q, k, v, scale=inp.scale, rows=np.arange(n))
    dt = time.perf_counter() - t0
    n = int(min(B * H * N, max(64, n * seconds / max(dt, 1e-3))))
    t0 = time.perf_counter()
    orc.attention(q, k, v, scale=inp.scale, rows=np.arange(n))
    dt = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(n * flops_per_row / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"first {n} query rows (of {B * H * N}) of the B{B} H{H} N{N} d{d} "
                      f"non-causal forward, fp64, {dt:.1f} s"}


def summarize(name, trace_dir, out):
    """Summary of rocprofv3 output for one workload's kernel: average kernel
    duration (--kernel-trace --stats), FETCH_SIZE / WRITE_SIZE per dispatch
    (--pmc runs) scaled by the same counters read on a plain copy of known
    size (the torch copy kernel run with --copy-calibration)."""
    import csv
    import glob
    kern = {"fwd": "attn_fwd_bf16", "fwd_causal": "attn_fwd_bf16", "softmax": "softmax_rows_resident",
            "softmax_2pass": "softmax_rows_streaming",
            "decode": "decode_split", "merge_lse": "merge_lse", "extend": "decode_split",
            "bwd": "attn_bwd_dkdv<false, 128>", "bwd_causal": "attn_bwd_dkdv<true, 128>",
            "fwd_fp8": "attn_fwd_fp8", "fwd_d64": "attn_fwd_bf16_d64", "bwd_d64": "attn_bwd_dkdv<false, 64>"}[name]
    lines = [f"# rocprofv3 summary: {name}", ""]
    trace = os.path.join(trace_dir, "trace", "run_kernel_trace.csv")
    avg_ns = None
    if os.path.exists(trace):
        # per (kernel, grid size): the attention kernel runs with different
        # grids for the non-causal and the causal workload
        groups = {}
        for r in csv.DictReader(open(trace)):
            short = r["Kernel_Name"].replace("osm::(anonymous namespace)::", "").replace("void ", "")
            short = short.split("(")[0]
            key = (short, int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"])))
            groups.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        lines += ["## kernel trace (--kernel-trace --stats): per kernel and grid", "",
                  "| kernel | workgroups | calls | avg us | min us | max us |", "|---|---|---|---|---|---|"]
        for (short, wg), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
            lines.append(f"| {short} | {wg} | {len(d)} | {sum(d) / len(d) / 1e3:.1f} | "
                         f"{min(d) / 1e3:.1f} | {max(d) / 1e3:.1f} |")
        # both head-dim-128 forwards run on persistent grids (one workgroup
        # per compute unit): the full-length one walks equal blocks, the
        # causal varlen one a schedule built from the lengths; head dim 64
        # runs one block per workgroup
        # (the piece kernel's grid is (pieces, kv heads, batch): 128 pieces
        # for decode, 8 for extend; the backward's key-major kernel is
        # instantiated for the causal mask or not)
        want = {"fwd": ("attn_fwd_bf16_d128_persist", None), "fwd_causal": ("attn_fwd_bf16_d128_sched", None),
                "softmax": ("softmax_rows_resident", None), "softmax_2pass": ("softmax_rows_streaming", None),
                "decode": ("decode_split", 128),
                "merge_lse": ("merge_lse", None), "extend": ("decode_split", 8),
                "bwd": ("attn_bwd_dkdv<false, 128>", None), "bwd_causal": ("attn_bwd_dkdv<true, 128>", None),
                "fwd_fp8": ("attn_fwd_fp8", None), "fwd_d64": ("attn_fwd_bf16_d64", None),
                "bwd_d64": ("attn_bwd_dkdv<false, 64>", None)}[name]
        for (short, wg), d in groups.items():
            if want[0] in short and (want[1] is None or wg == want[1]):
                avg_ns = sum(d) / len(d)
        lines.append("")
    counters = {}
    pmc_ns = []    # kernel durations of the counter runs' dispatches
    for f in sorted(glob.glob(os.path.join(trace_dir, "pmc_*", "run_counter_collection.csv"))):
        per = {}
        for r in csv.DictReader(open(f)):
            if kern in r["Kernel_Name"] and r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                pmc_ns.append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
            # the calibration copy is torch's device-to-device copy_, which
            # runs the HIP runtime's buffer-copy kernel
            key = ("copy" if "copyBuffer" in r["Kernel_Name"]
                   else ("kernel" if kern in r["Kernel_Name"] else None))
            if key is None:
                continue
            per.setdefault((key, r["Counter_Name"]), {}).setdefault(r["Dispatch_Id"], 0.0)
            per[(key, r["Counter_Name"])][r["Dispatch_Id"]] += float(r["Counter_Value"])
        for k, d in per.items():
            # the calibration copy is the largest buffer copy of the run
            # (small ones upload lengths); the kernel is averaged
            counters[k] = max(d.values()) if k[0] == "copy" else sum(d.values()) / len(d)
    cal = None
    if counters:
        lines += ["## counters per dispatch (--pmc)", "", "| kernel | counter | value (FETCH_SIZE, WRITE_SIZE in KiB) |",
                  "|---|---|---|"]
        for (k, c), v in sorted(counters.items()):
            lines.append(f"| {k} | {c} | {v:.0f} |")
        lines.append("")
    copy_bytes = None
    for f in glob.glob(os.path.join(trace_dir, "copy_bytes.txt")):
        copy_bytes = float(open(f).read().strip())
    traffic = None
    if copy_bytes and ("copy", "FETCH_SIZE") in counters and ("kernel", "FETCH_SIZE") in counters:
        f_scale = copy_bytes / (counters[("copy", "FETCH_SIZE")] * 1024)
        w_scale = copy_bytes / (counters[("copy", "WRITE_SIZE")] * 1024) if ("copy", "WRITE_SIZE") in counters else f_scale
        traffic = (counters[("kernel", "FETCH_SIZE")] * 1024 * f_scale
                   + counters.get(("kernel", "WRITE_SIZE"), 0.0) * 1024 * w_scale)
        lines += [f"copy calibration: {copy_bytes:.0f} bytes read and written by the copy; "
                  f"FETCH_SIZE scale {f_scale:.4f}, WRITE_SIZE scale {w_scale:.4f}", ""]
    kc = {c: v for (k, c), v in counters.items() if k == "kernel"}
    if "SQ_VALU_MFMA_BUSY_CYCLES" in kc and "GRBM_GUI_ACTIVE" in kc and pmc_ns:
        # GRBM_GUI_ACTIVE is summed over the 8 XCDs; SQ_VALU_MFMA_BUSY_CYCLES over
        # the 1024 SIMDs, in cycles of the matrix pipe at its full issue rate
        cycles = kc["GRBM_GUI_ACTIVE"] / 8
        busy = kc["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024
        ns = sum(pmc_ns) / len(pmc_ns)
        lines += [f"engine clock over the kernel: {cycles / ns:.2f} GHz (GRBM_GUI_ACTIVE per XCD / {ns / 1e3:.1f} us)",
                  f"MFMA busy: {100 * busy / cycles:.1f}% of the kernel's cycles per SIMD "
                  f"(SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / cycles)"]
        for c, per, what in (("SQ_INSTS_VALU_MFMA_MOPS_BF16", 512, "bf16"), ("SQ_INSTS_VALU_MFMA_MOPS_F8", 512, "fp8")):
            if c in kc and kc[c] > 0:
                lines.append(f"{what} MFMA flops executed per launch: {kc[c] * per:.4e} ({c} x {per})")
        lines.append("")
    if "SQ_INSTS_MFMA" in kc and kc["SQ_INSTS_MFMA"] > 0:
        # instruction mix per matrix instruction (all counts are per wave
        # instruction; SQ_INSTS_VALU includes the MFMA instructions themselves)
        nm = kc["SQ_INSTS_MFMA"]
        mix = []
        if "SQ_INSTS_VALU" in kc:
            mix.append(f"other VALU {(kc['SQ_INSTS_VALU'] - nm) / nm:.2f}")
        mix += [f"{what} {kc[c] / nm:.2f}" for c, what in
                (("SQ_INSTS_VALU_TRANS_F32", "of them exp (TRANS_F32)"), ("SQ_INSTS_LDS", "LDS"), ("SQ_INSTS_SALU", "SALU"))
                if c in kc]
        lines.append(f"per MFMA instruction ({nm:.4e} per launch): " + ", ".join(mix))
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in kc and "SQ_VALU_MFMA_BUSY_CYCLES" in kc:
            lines.append(f"MFMA cycles with VALU co-executing: "
                         f"{100 * kc['SQ_VALU_MFMA_COEXEC_CYCLES'] / kc['SQ_VALU_MFMA_BUSY_CYCLES']:.1f}%")
        if "SQ_LDS_BANK_CONFLICT" in kc and "SQ_LDS_IDX_ACTIVE" in kc and kc["SQ_LDS_IDX_ACTIVE"] > 0:
            lines.append(f"LDS bank conflicts: {kc['SQ_LDS_BANK_CONFLICT'] / kc['SQ_LDS_IDX_ACTIVE']:.4f} "
                         f"of LDS active cycles (SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE)")
        lines.append("")
    if "SQ_WAVE_CYCLES" in kc and kc["SQ_WAVE_CYCLES"] > 0:
        wc = kc["SQ_WAVE_CYCLES"]
        part = [f"{c[3:]}: {100 * kc[c] / wc:.1f}%" for c in
                ("SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS",
                 "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY") if c in kc]
        lines += ["share of wave cycles (SQ_WAVE_CYCLES): " + ", ".join(part), ""]
    lines += [f"kernel_source_sha256_16: {source_hash(name)}",
              f"avg_kernel_us: {avg_ns / 1e3:.2f}" if avg_ns else "avg_kernel_us: null",
              f"traffic_bytes_per_launch: {traffic:.0f}" if traffic else "traffic_bytes_per_launch: null", ""]
    cmdf = os.path.join(trace_dir, "commands.txt")
    if os.path.exists(cmdf):
        lines += ["## commands", "", "```", open(cmdf).read().strip(), "```", ""]
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))
    return 0


def sweep(args):
    """The forward (osm_attn_fwd), or with --sweep-bwd the backward
    (osm_attn_bwd, from the forward's O and LSE and an N(0, 1) output
    gradient), over sequence lengths 1K-32K at a fixed 16384 tokens per head
    group (B = 16384 / N), head dims 128 (32 heads) and 64 (64 heads), full
    length, causal or not; inputs N(0, 1) rounded to bf16, drawn on the
    device from a seeded generator.  One JSON line per configuration: median
    and minimum of the timed calls (HIP events on the current stream) and
    TFLOP/s of the median against the bf16 peak (4 N^2 d flop per head for
    the forward, 10 N^2 d for the backward; halved, plus the diagonal, with
    the causal mask)."""
    import torch
    import exact_attention_online_softmax_amd as osm

    osm.load_library()
    torch.cuda.set_device(0)
    for d, H in ((128, 32), (64, 64)):
        for causal in (False, True):
            for N in (1024, 2048, 4096, 8192, 16384, 32768):
                B = max(1, 16384 // N)
                gen = torch.Generator(device="cuda").manual_seed(7000 + N + d + causal)
                q, k, v = (torch.randn((B, H, N, d), generator=gen, device="cuda").to(torch.bfloat16)
                           for _ in range(3))
                o = torch.empty_like(q)
                lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
                call = lambda: osm.attn_fwd(q, k, v, causal=causal, out=o, lse=lse)
                if args.sweep_bwd:
                    call()
                    do = torch.randn((B, H, N, d), generator=gen, device="cuda").to(torch.bfloat16)
                    ws = torch.empty(osm.attn_bwd_workspace_bytes(B, H, N), dtype=torch.uint8, device="cuda")
                    grads = [torch.empty_like(q) for _ in range(3)]
                    call = lambda: osm.attn_bwd(q, k, v, o, lse, do, causal=causal, workspace=ws,
                                                dq=grads[0], dk=grads[1], dv=grads[2])
                for _ in range(args.warmup):
                    call()
                ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in range(args.steps)]
                torch.cuda.synchronize()
                for a, b in ev:
                    a.record()
                    call()
                    b.record()
                torch.cuda.synchronize()
                ms = sorted(a.elapsed_time(b) for a, b in ev)
                med = ms[len(ms) // 2]
                pairs = B * H * (N * (N + 1) / 2 if causal else N * N)
                tf = (10.0 if args.sweep_bwd else 4.0) * d * pairs / (med / 1e3) / 1e12
                print(json.dumps({"sweep": "attn_bwd" if args.sweep_bwd else "attn_fwd", "head_dim": d, "causal": causal, "batch": B, "heads": H,
                                  "seq_len": N, "ms_median": round(med, 4), "ms_min": round(ms[0], 4),
                                  "tflops": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4)}), flush=True)
                del q, k, v, o, lse, call
                if args.sweep_bwd:
                    del do, ws, grads
    return 0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--only", choices=WORKLOADS, default=None,
                    help="run one operation only (for profiling)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the reference copy and matrix-core kernels")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of MIB MiB per step (scales rocprof "
                         "FETCH_SIZE/WRITE_SIZE to bytes)")
    ap.add_argument("--sweep-bwd", action="store_true",
                    help="with --sweep: the backward instead of the forward")
    ap.add_argument("--sweep", action="store_true",
                    help="the forward over sequence lengths and head dims (one JSON line each)")
    ap.add_argument("--summarize", nargs=3, metavar=("NAME", "TRACE_DIR", "OUT"), default=None,
                    help="write a profile summary from rocprofv3 CSV output: NAME is a workload "
                         "name, TRACE_DIR holds run_kernel_stats.csv and pmc_*/ counter dirs")
    args = ap.parse_args()
    if args.summarize:
        return summarize(*args.summarize)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(attention shards by batch and head with no exchange between GPUs)", file=sys.stderr)
        return 2
    if args.sweep:
        return sweep(args)

    import torch
    import exact_attention_online_softmax_amd as osm
    from exact_attention_online_softmax_amd import inputs

    osm.load_library()
    torch.cuda.set_device(0)
    names = list(WORKLOADS) if args.only is None else [args.only]
    calls, work = {}, {}

    if "softmax" in names:
        log("inputs: softmax 4096 x 32000")
        x = torch.from_numpy(inputs.config2()).to("cuda")
        y = torch.empty_like(x)
        calls["softmax"] = lambda: osm.softmax_rows(x, out=y)
        # one HBM read + one HBM write per element: the row stays in registers
        work["softmax"] = ("hbm", 8.0 * x.numel(), "4096 x 32000 fp32, 8 B/elem")
    if "softmax_2pass" in names:
        if "softmax" not in names:
            log("inputs: softmax 4096 x 32000")
            x = torch.from_numpy(inputs.config2()).to("cuda")
        y2 = torch.empty_like(x)
        calls["softmax_2pass"] = lambda: osm.softmax_rows(x, out=y2, two_pass=True)
        # the pages' count: two loads and one store per element
        work["softmax_2pass"] = ("hbm", 12.0 * x.numel(), "4096 x 32000 fp32, two passes, 12 B/elem")
    if "fwd" in names or "bwd" in names or args.only is None:
        log("inputs: fwd B4 H32 N4096 d128")
        inp3 = inputs.config3()
        q3, k3, v3 = (bf16_dev(a, torch) for a in (inp3.q, inp3.k, inp3.v))
        o3 = torch.empty_like(q3)
        l3 = torch.empty(q3.shape[:3], dtype=torch.float32, device="cuda")
        B, H, N, d = q3.shape
        if "fwd" in names:
            calls["fwd"] = lambda: osm.attn_fwd(q3, k3, v3, scale=inp3.scale, out=o3, lse=l3)
            work["fwd"] = ("mfma", 4.0 * B * H * N * N * d, "B4 H32 N4096 d128 non-causal")
        if "bwd" in names:
            log("inputs: bwd B4 H32 N4096 d128, output gradient")
            osm.attn_fwd(q3, k3, v3, scale=inp3.scale, out=o3, lse=l3)
            do3 = bf16_dev(inputs.output_grad(4, 32, 4096, 128, inputs.SEED_BASE + 8), torch)
            ws3 = torch.empty(osm.attn_bwd_workspace_bytes(4, 32, 4096), dtype=torch.uint8, device="cuda")
            g3 = [torch.empty_like(t) for t in (q3, k3, v3)]
            calls["bwd"] = lambda: osm.attn_bwd(q3, k3, v3, o3, l3, do3, scale=inp3.scale, workspace=ws3,
                                                dq=g3[0], dk=g3[1], dv=g3[2])
            # five products per (query, key) pair: S again, dP, dV, dQ, dK
            work["bwd"] = ("mfma", 10.0 * B * H * N * N * d, "backward of B4 H32 N4096 d128 non-causal")
    if "fwd_d64" in names or "bwd_d64" in names:
        log("inputs: fwd B4 H64 N4096 d64")
        inp64 = inputs.attention_inputs(4, 64, 64, 4096, 4096, 64, seed=inputs.SEED_BASE + 11)
        q64, k64, v64 = (bf16_dev(a, torch) for a in (inp64.q, inp64.k, inp64.v))
        o64 = torch.empty_like(q64)
        l64 = torch.empty(q64.shape[:3], dtype=torch.float32, device="cuda")
        scale64 = inp64.scale
        calls["fwd_d64"] = lambda: osm.attn_fwd(q64, k64, v64, scale=scale64, out=o64, lse=l64)
        work["fwd_d64"] = ("mfma", 4.0 * 4 * 64 * 4096 * 4096 * 64, "B4 H64 N4096 d64 non-causal")
        if "bwd_d64" in names:
            log("inputs: bwd B4 H64 N4096 d64, output gradient")
            calls["fwd_d64"]()
            do64 = bf16_dev(inputs.output_grad(4, 64, 4096, 64, inputs.SEED_BASE + 12), torch)
            ws64 = torch.empty(osm.attn_bwd_workspace_bytes(4, 64, 4096), dtype=torch.uint8, device="cuda")
            g64 = [torch.empty_like(t) for t in (q64, k64, v64)]
            calls["bwd_d64"] = lambda: osm.attn_bwd(q64, k64, v64, o64, l64, do64, scale=scale64,
                                                    workspace=ws64, dq=g64[0], dk=g64[1], dv=g64[2])
            work["bwd_d64"] = ("mfma", 10.0 * 4 * 64 * 4096 * 4096 * 64,
                               "backward of B4 H64 N4096 d64 non-causal")
        if "fwd_d64" not in names:
            del calls["fwd_d64"], work["fwd_d64"]
        del inp64
    if "fwd_causal" in names or "bwd_causal" in names:
        log("inputs: fwd causal B8 H16 N8192 d128 varlen")
        inp4 = inputs.config4()
        q4, k4, v4 = (bf16_dev(a, torch) for a in (inp4.q, inp4.k, inp4.v))
        o4 = torch.empty_like(q4)
        l4 = torch.empty(q4.shape[:3], dtype=torch.float32, device="cuda")
        lens4 = torch.from_numpy(inp4.seqlens_q).to("cuda")
        scale4 = inp4.scale
        calls["fwd_causal"] = lambda: osm.attn_fwd(q4, k4, v4, scale=scale4, causal=True,
                                                   seqlens_q=lens4, seqlens_k=lens4, out=o4, lse=l4)
        Lb = inp4.seqlens_q.astype(np.float64)
        pairs4 = 128 * 16 * float(np.sum(Lb * (Lb + 1) / 2))
        work["fwd_causal"] = ("mfma", 4.0 * pairs4, "B8 H16 N8192 d128 causal, L_b U[1024,8192]")
        if "bwd_causal" in names:
            log("inputs: bwd causal, output gradient")
            calls["fwd_causal"]()
            do4 = bf16_dev(inputs.output_grad(8, 16, 8192, 128, inputs.SEED_BASE + 9,
                                              seqlens_q=inp4.seqlens_q, poison=True), torch)
            ws4 = torch.empty(osm.attn_bwd_workspace_bytes(8, 16, 8192), dtype=torch.uint8, device="cuda")
            g4 = [torch.empty_like(t) for t in (q4, k4, v4)]
            calls["bwd_causal"] = lambda: osm.attn_bwd(q4, k4, v4, o4, l4, do4, scale=scale4, causal=True,
                                                       seqlens_q=lens4, seqlens_k=lens4, workspace=ws4,
                                                       dq=g4[0], dk=g4[1], dv=g4[2])
            # five products per visible (query, key) pair: S again, dP, dV, dQ, dK
            work["bwd_causal"] = ("mfma", 10.0 * pairs4,
                                  "backward of B8 H16 N8192 d128 causal, L_b U[1024,8192]")
        del inp4
    if "decode" in names:
        log("inputs: decode B16 Hq32 Hkv8 L<=32768 d128")
        inp5 = inputs.config5()
        q5 = bf16_dev(inp5.q[:, :, 0, :], torch)
        k5, v5 = bf16_dev(inp5.k, torch), bf16_dev(inp5.v, torch)
        lens5 = torch.from_numpy(inp5.seqlens_k).to("cuda")
        ws5 = torch.empty(osm.decode_workspace_bytes(16, 32, 32768, 128, 256), dtype=torch.uint8,
                          device="cuda")
        o5 = torch.empty_like(q5)
        l5 = torch.empty((16, 32), dtype=torch.float32, device="cuda")
        scale5 = inp5.scale
        calls["decode"] = lambda: osm.attn_decode_splitkv(q5, k5, v5, lens5, scale=scale5,
                                                          split_size=256, workspace=ws5, out=o5,
                                                          lse=l5)
        Lb = inp5.seqlens_k.astype(np.float64)
        pieces = np.ceil(Lb / 256)
        kv = float(np.sum(Lb)) * 8 * 128 * 2 * 2
        io = 16 * 32 * 128 * 2 * 2 + 16 * 32 * 4
        partials = 2.0 * float(np.sum(pieces)) * 32 * (128 + 2) * 4
        work["decode"] = ("hbm", kv + io + partials, "B16 Hq32 Hkv8 d128, L_b U[4096,32768], split 256")
        del inp5

    if "merge_lse" in names:
        log("inputs: merge_lse 8 pieces x 524288 rows x d128 bf16")
        S6, R6, D6 = 8, 4 * 32 * 4096, 128
        o6, l6 = inputs.lse_parts(S6, R6, D6, inputs.SEED_BASE + 6, dtype="bf16")
        op6 = bf16_dev(o6, torch)
        lp6 = torch.from_numpy(l6).to("cuda")
        del o6, l6
        out6 = torch.empty((R6, D6), dtype=torch.bfloat16, device="cuda")
        lse6 = torch.empty(R6, dtype=torch.float32, device="cuda")
        calls["merge_lse"] = lambda: osm.merge_lse(op6, lp6, out=out6, lse=lse6)
        work["merge_lse"] = ("hbm", float(S6 * R6 * (D6 * 2 + 4) + R6 * (D6 * 2 + 4)),
                             "8 pieces of the B4 H32 N4096 d128 output (524288 rows), bf16")

    if "extend" in names:
        log("inputs: extend B16 Hq32 Hkv8 d128 bf16, 4096 new keys per call")
        B7, Hq7, Hkv7, N7, D7 = 16, 32, 8, 4096, 128
        inp7 = inputs.attention_inputs(B7, Hq7, Hkv7, 1, N7, D7, inputs.SEED_BASE + 7)
        q7 = bf16_dev(inp7.q[:, :, 0, :], torch)
        k7, v7 = bf16_dev(inp7.k, torch), bf16_dev(inp7.v, torch)
        state7 = osm.attn_state(B7, Hq7, D7)
        ws7 = torch.empty(osm.decode_workspace_bytes(B7, Hq7, N7, D7, 512), dtype=torch.uint8, device="cuda")
        scale7 = inp7.scale
        del inp7
        calls["extend"] = lambda: osm.attn_extend(q7, k7, v7, state7, scale=scale7, split_size=512,
                                                  workspace=ws7)
        pieces7 = N7 // 512
        work["extend"] = ("hbm", float(B7 * Hkv7 * N7 * D7 * 2 * 2 + B7 * Hq7 * D7 * 2
                                       + 2 * B7 * Hq7 * (D7 + 2) * 4 + 2 * B7 * Hq7 * pieces7 * (D7 + 2) * 4),
                          "B16 Hq32 Hkv8 d128 bf16, 4096 new keys folded into a persisted state")

    if "fwd_fp8" in names:
        log("inputs: fwd fp8 B4 H32 N4096 d128 (E4M3 codes)")
        inp8 = inputs.attention_inputs(4, 32, 32, 4096, 4096, 128, seed=inputs.SEED_BASE + 10, dtype="fp8")
        q8, k8, v8 = (torch.from_numpy(a).to("cuda") for a in (inp8.q, inp8.k, inp8.v))
        o8 = torch.empty(q8.shape, dtype=torch.bfloat16, device="cuda")
        l8 = torch.empty(q8.shape[:3], dtype=torch.float32, device="cuda")
        scale8 = inp8.scale
        calls["fwd_fp8"] = lambda: osm.attn_fwd_fp8(q8, k8, v8, scale=scale8, out=o8, lse=l8)
        work["fwd_fp8"] = ("mfma8", 4.0 * 4 * 32 * 4096 * 4096 * 128, "B4 H32 N4096 d128 non-causal, E4M3 Q/K/V")
        del inp8

    if args.copy_calibration:
        n = args.copy_calibration * 1024 * 1024 // 4
        csrc = torch.ones(n, dtype=torch.float32, device="cuda")
        cdst = torch.empty_like(csrc)
        names.append("copy")
        calls["copy"] = lambda: cdst.copy_(csrc)
        work["copy"] = ("hbm", 8.0 * n, f"device copy {args.copy_calibration} MiB")

    # ---- warmup, then K timed steps --------------------------------------
    for _ in range(args.warmup):
        for n in names:
            calls[n]()
    torch.cuda.synchronize()
    ev = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)] for n in names}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        for n in names:
            a, b = ev[n][s]
            a.record()
            calls[n]()
            b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    times = {n: [a.elapsed_time(b) for a, b in ev[n]] for n in names}
    ms = {n: float(np.mean(times[n])) for n in names}

    comps = {}
    for n in names:
        bound, amount, desc = work[n]
        t = ms[n] / 1e3
        if bound == "mfma":
            ach, peak, unit = amount / t / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
        elif bound == "mfma8":
            ach, peak, unit = amount / t / 1e12, PEAK_FP8_TFLOPS, "TFLOP/s"
        else:
            ach, peak, unit = amount / t / 1e9, PEAK_HBM_GBS, "GB/s"
        comps[n] = {"workload": desc, "ms": round(ms[n], 4), "ms_median": round(float(np.median(times[n])), 4),
                    "ms_min": round(float(np.min(times[n])), 4), "achieved": round(ach, 2),
                    "unit": unit, "bound": "hbm" if bound == "hbm" else "mfma",
                    "peak": round(peak, 1), "frac": round(ach / peak, 4),
                    "algorithmic": amount}
        if bound == "mfma8":
            comps[n]["dtype"] = "fp8"
    head = "fwd" if "fwd" in comps else names[0]
    hc = comps[head]
    roofline = {"bound": hc["bound"], "achieved": hc["achieved"], "peak": hc["peak"],
                "unit": hc["unit"], "frac": hc["frac"],
                "traffic": traffic_from_profile(PROFILE_FWD, "fwd") if head == "fwd" else None}
    out = {"metric": METRIC, "value": hc["achieved"], "unit": hc["unit"], "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(wall * 1e3 / args.steps, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"attn_fwd {hc['workload']}" if head == "fwd" else hc["workload"],
                      "step": "softmax_rows + softmax_rows_twopass + attn_fwd (non-causal) + attn_fwd (causal varlen) "
                              "+ attn_decode_splitkv + merge_lse + attn_extend + attn_bwd (non-causal) "
                              "+ attn_bwd (causal varlen) + attn_fwd_fp8 + attn_fwd (head dim 64) "
                              "+ attn_bwd (head dim 64)" if args.only is None
                              else args.only,
                      "global_batch": 4, "seq_len": 4096, "parallelism": "none (1 GPU)"},
           "roofline": roofline, "components": comps}
    if not args.no_context and args.only is None:
        log("context: reference copy and matrix-core kernels")
        out["achievable"] = achievable(torch)
    if not args.no_cpu_baseline and args.only is None:
        log("cpu baseline: oracle on a sample of the headline workload")
        out["cpu_baseline"] = cpu_baseline(inp3, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
