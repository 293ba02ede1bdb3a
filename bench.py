"""Benchmark of the attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch of synthetic input:
for the default workload (causal, B=4, H=16, N=4096, d=128) that is the
forward (fa_fwd) and the three backward stages (fa_bwd_preprocess,
fa_bwd_dkdv, fa_bwd_dq).  Forward-only workloads run fa_fwd (or
fa_fwd_f32 / fa_fwd_kvlen / fa_fwd_block_sparse); the FP8 workload runs
fa_fp8_quantize then fa_fwd_fp8_quantized on the bf16 inputs (its roofline is
the attention kernel against the fp8 matrix peak); the linear-attention
workload runs fa_linear_fwd (HBM roofline).  Inputs are resident in HBM
before timing starts.

Throughput is algorithmic: 4d FLOP per visible (query, key) pair for the
forward and 10d for the backward (causal: N(N+1)/2 pairs per head); masked
work, exp and max/sum operations are not counted, and neither is the
backward's second recomputation of S and dP in fa_bwd_dq (the backward
kernels execute 14d per pair).  The roofline's dominant kernel is fa_bwd_dkdv
(8d per pair) for forward+backward workloads and fa_fwd otherwise.  Rank 0 prints one JSON
line with a "roofline" object for the dominant kernel (its average launch
duration from HIP events recorded on the launch stream during the timed
steps) and a "cpu_baseline" object (the fp64 oracle timed on a bounded
sample of heads on the host cores).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synthetic as S  # noqa: E402

METRIC = ("attention fwd(+bwd) TFLOP/s bf16 causal, N=1K-23.4K; "
          "% of MFMA peak")
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 matrix peak (published)
PEAK_F32_TFLOPS = 157.3         # MI355X fp32 matrix peak (published)
PEAK_FP8_TFLOPS = 5000.0        # MI355X dense fp8 matrix peak (published)
DEFAULT_WORKLOAD = "causal_fwd_bwd_d128"
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "traffic.json")


def _sources_digest(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "io_aware_tiled_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def visible_pairs(w: S.Workload, kv_len, block_mask=None) -> int:
    if block_mask is not None:
        # kept 256x128 blocks of each head (every batch entry), causal pairs
        # counted inside diagonal blocks
        i = np.arange(w.N)[:, None]
        j = np.arange(w.N)[None, :]
        total = 0
        for h in range(block_mask.shape[0]):
            vis = block_mask[h].astype(bool)[i // 256, j // 128]
            if w.causal:
                vis &= j <= i
            total += int(vis.sum())
        return total * w.B
    if w.causal:
        per = w.N * (w.N + 1) // 2
        return per * w.B * w.H
    if kv_len is None:
        return w.N * w.N * w.B * w.H
    return int(sum(w.N * min(max(int(L), 0), w.N) for L in kv_len)) * w.H


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def cpu_baseline(w: S.Workload, inp: dict, target_s: float = 15.0) -> dict:
    """Time the fp64 oracle (as it stands) on a bounded sample of heads."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    nh = 1
    # one head first, then grow the sample toward target_s of CPU work
    sl = (slice(0, 1), slice(0, nh))
    q, k, v = (inp[n][sl] for n in ("q", "k", "v"))
    kv = None if inp["kv_len"] is None else inp["kv_len"][:1]
    bm = inp.get("block_mask")
    import oracle.dropout
    import oracle.fp8
    import oracle.linear
    dr = inp.get("dropout")

    def run(q, k, v, nh, sl):
        if dr is not None:
            p8 = oracle.dropout.threshold(dr["p"])
            oracle.dropout.attention_dropout_fwd(q, k, v, inp["scale"],
                                                 inp["causal"], p8, dr["seed"],
                                                 dr["offset"])
            if w.backward:
                oracle.dropout.attention_dropout_bwd(
                    q, k, v, inp["do"][sl], inp["scale"], inp["causal"], p8,
                    dr["seed"], dr["offset"])
            return
        if w.linear:
            oracle.linear.linear_attention_fwd(q, k, v, inp["scale"])
            return
        if inp.get("signs") is not None:
            oracle.fp8.fp8_forward(q, k, v, inp["scale"], inp["causal"],
                                   inp["signs"], workers=cores)
            return
        oracle.attention_fwd(q, k, v, inp["scale"], inp["causal"], kv,
                             workers=cores,
                             block_mask=None if bm is None else bm[:nh].astype(bool))
        if w.backward:
            oracle.attention_bwd(q, k, v, inp["do"][sl], inp["scale"],
                                 inp["causal"], kv, workers=cores,
                                 block_mask=None if bm is None
                                 else bm[:nh].astype(bool))
    t0 = time.perf_counter()
    run(q, k, v, nh, sl)
    t1 = time.perf_counter() - t0
    nh = int(max(1, min(w.H, cores, target_s // max(t1, 1e-3))))
    if nh > 1:
        sl = (slice(0, 1), slice(0, nh))
        q, k, v = (inp[n][sl] for n in ("q", "k", "v"))
        t0 = time.perf_counter()
        run(q, k, v, nh, sl)
        t1 = time.perf_counter() - t0
    sw = S.Workload(w.name, 1, nh, w.N, w.d, w.dtype, w.causal, w.seeds,
                    w.backward)
    pairs = visible_pairs(sw, kv, None if bm is None else bm[:nh])
    flops = pairs * w.d * (4 + (10 if w.backward else 0))
    if w.linear:
        flops = linear_flops(S.Workload(w.name, 1, nh, w.N, w.d, w.dtype, True,
                                        w.seeds, linear=True))
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    if w.linear:
        what = "fp64 numpy causal linear attention (quadratic definition)"
    elif inp.get("signs") is not None:
        what = ("fp64 numpy model of the FP8 path (rotation, block "
                "quantisation, fp64 attention), forward")
    elif dr is not None:
        what = ("fp64 numpy oracle with dropout (Philox keep mask), "
                + ("forward+backward" if w.backward else "forward"))
    else:
        what = ("fp64 numpy oracle, "
                + ("forward+backward" if w.backward else "forward"))
    return {"value": flops / t1 / 1e12, "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle", "cpu_model": model, "blas_threads": cores,
            "sample": (what +
                       f" of batch 0, heads 0..{nh - 1} of {w.name} "
                       f"(N={w.N}, d={w.d}); {t1:.2f} s; {cores} threads "
                       + ("(BLAS pool; heads in sequence)" if dr is not None
                          else "(BLAS pool + one worker thread per head)"))}


# rocprofv3 kernel-name fragment -> bench step (all variants of a step)
KERNEL_KEYS = (("bwd_dkdv_", "bwd_dkdv"), ("bwd_dq_", "bwd_dq"),
               ("bwd_preprocess_", "bwd_preprocess"),
               ("fwd_bf16_", "fwd"), ("fwd_f32_", "fwd"),
               ("fwd_fp8_", "fwd_fp8"), ("fp8_quant_", "fp8_quantize"),
               ("linear_fwd_", "linear_fwd"))
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E bandwidth (published)
LINEAR_CHUNK = 64


def linear_flops(w: S.Workload) -> float:
    """Algorithmic FLOPs of chunkwise causal linear attention: 4d per
    visible (query, key) pair inside a 64-row chunk (Q K^T and A V), plus
    2d^2 per row for Q S and 2d^2 per row for the state update K^T V."""
    full, rem = divmod(w.N, LINEAR_CHUNK)
    intra = full * LINEAR_CHUNK * (LINEAR_CHUNK + 1) // 2 + rem * (rem + 1) // 2
    return w.B * w.H * (4.0 * w.d * intra + 4.0 * w.N * w.d * w.d)


def fp8_workspace_bytes(w: S.Workload) -> int:
    """Quantised Q, K (rows of 144 or 80 bytes) and V (80 bytes per channel
    per 64 keys) of the FP8 path."""
    np_ = -(-w.N // 64) * 64
    rb = 144 if w.d == 128 else 80
    return 2 * w.B * w.H * np_ * rb + w.B * w.H * (np_ // 64) * w.d * 80


def algorithmic_bytes(w: S.Workload, kernel: str) -> int:
    """Bytes a kernel must move to and from HBM at least once: its inputs and
    outputs, each read or written exactly once."""
    el = 4 if w.dtype == "f32" else 2
    t = w.B * w.H * w.N * w.d * el          # one [B,H,N,d] tensor
    r = w.B * w.H * w.N * 4                 # one float32 [B,H,N] row vector
    if kernel == "fp8_quantize":                 # Q,K,V -> workspace
        return 3 * t + fp8_workspace_bytes(w)
    if kernel == "fwd_fp8":                      # workspace -> O, LSE
        return fp8_workspace_bytes(w) + t + r
    if kernel == "linear_fwd":                   # Q,K,V -> O
        return 4 * t
    return {"fwd": 3 * t + t + r,             # Q,K,V -> O, LSE
            "bwd_preprocess": 2 * t + r,      # O, dO -> D
            "bwd_dkdv": 4 * t + 2 * r + 2 * t,  # Q,K,V,dO,LSE,D -> dK,dV
            "bwd_dq": 4 * t + 2 * r + t}[kernel]  # Q,K,V,dO,LSE,D -> dQ


def _pmc_per_kernel(path, counter):
    """Average counter value per dispatch, keyed by kernel short name."""
    import csv
    vals = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            key = None
            for frag, k in KERNEL_KEYS:
                if "fa::" in name and frag in name:
                    key = k
            if "neg_kernel" in name:
                key = "copy_calibration"
            if key is not None:
                vals.setdefault(key, []).append(float(r["Counter_Value"]))
    return {k: (float(np.mean(v)), len(v)) for k, v in vals.items()}


def write_traffic(w: S.Workload, csvs, command, mib) -> int:
    fetch = _pmc_per_kernel(csvs[0], "FETCH_SIZE")
    write = _pmc_per_kernel(csvs[1], "WRITE_SIZE")
    if "copy_calibration" not in fetch or "copy_calibration" not in write:
        print("no calibration kernel in the counter files", file=sys.stderr)
        return 1
    # The calibration dispatch reads and writes mib MiB.
    cal_bytes = mib * (1 << 20)
    f_scale = cal_bytes / (fetch["copy_calibration"][0] * 1024.0)
    w_scale = cal_bytes / (write["copy_calibration"][0] * 1024.0)
    src = {"fwd": ["fa_fwd.hip", "fa_common.h"],
           "linear_fwd": ["fa_linear.hip", "fa_common.h"],
           "fwd_fp8": ["fa_fp8.hip", "fa_common.h"],
           "fp8_quantize": ["fa_fp8.hip", "fa_common.h"]}
    entry = {}
    for k in fetch:
        if k == "copy_calibration" or k not in write:
            continue
        fb = fetch[k][0] * 1024.0 * f_scale
        wb = write[k][0] * 1024.0 * w_scale
        entry[k] = {
            "fetch_bytes_per_launch": round(fb), "write_bytes_per_launch": round(wb),
            "bytes_per_launch": round(fb + wb),
            "algorithmic_bytes_per_launch": algorithmic_bytes(w, k),
            "dispatches": fetch[k][1],
            "source_digest": _sources_digest(src.get(k, ["fa_bwd.hip", "fa_common.h"])),
        }
    tr = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
    tr[w.name] = {"kernels": entry, "command": command,
                  "calibration": {"bytes": cal_bytes,
                                  "fetch_kib_measured": fetch["copy_calibration"][0],
                                  "write_kib_measured": write["copy_calibration"][0],
                                  "fetch_scale": f_scale, "write_scale": w_scale}}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(tr, f, indent=1, sort_keys=True)
    md = os.path.join(PROFILES, f"traffic_{w.name}.md")
    with open(md, "w") as f:
        f.write(f"# HBM traffic per launch: {w.name} (B={w.B} H={w.H} N={w.N} "
                f"d={w.d}, causal={w.causal})\n\nCommands (repository root, one "
                f"MI355X):\n\n```\n{command}\n```\n\n"
                "FETCH_SIZE and WRITE_SIZE (KiB per dispatch) scaled by the "
                f"calibration copy of {mib} MiB: fetch x{f_scale:.4f}, write "
                f"x{w_scale:.4f} (measured {fetch['copy_calibration'][0]:.0f} / "
                f"{write['copy_calibration'][0]:.0f} KiB).\n\n"
                "| kernel | fetch MB | write MB | total MB | algorithmic MB | "
                "total / algorithmic |\n|---|---|---|---|---|---|\n")
        for k, e in sorted(entry.items()):
            f.write(f"| {k} | {e['fetch_bytes_per_launch']/1e6:.1f} | "
                    f"{e['write_bytes_per_launch']/1e6:.1f} | "
                    f"{e['bytes_per_launch']/1e6:.1f} | "
                    f"{e['algorithmic_bytes_per_launch']/1e6:.1f} | "
                    f"{e['bytes_per_launch']/e['algorithmic_bytes_per_launch']:.2f} |\n")
    print(open(md).read())
    return 0


def summarize_counters(w: S.Workload, csvs, command) -> int:
    """Per-kernel MFMA busy, executed MFMA FLOP, LDS bank conflicts and L2 hit
    rate from two rocprofv3 --pmc collections of a bench run."""
    vals = {}
    for path in csvs:
        import csv
        with open(path) as f:
            for r in csv.DictReader(f):
                name = r["Kernel_Name"]
                key = None
                for frag, k in KERNEL_KEYS:
                    if "fa::" in name and frag in name:
                        key = k
                if key is None:
                    continue
                vals.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(
                    float(r["Counter_Value"]))
                if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                    vals[key].setdefault("_ns", []).append(
                        float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
    ginp = S.make_inputs(w)
    pairs = visible_pairs(w, ginp["kv_len"], ginp.get("block_mask"))
    alg = {"fwd": 4 * w.d * pairs, "bwd_dkdv": 8 * w.d * pairs,
           "bwd_dq": 2 * w.d * pairs, "bwd_preprocess": 0}
    n_xcd, n_simd = 8, 1024
    md = os.path.join(PROFILES, f"counters_{w.name}.md")
    with open(md, "w") as f:
        f.write(f"# Hardware counters: {w.name} (B={w.B} H={w.H} N={w.N} d={w.d}, "
                f"causal={w.causal})\n\nCommands (repository root, one MI355X):"
                f"\n\n```\n{command}\n```\n\nPer dispatch (mean over the run's "
                "dispatches).  Kernel cycles = GRBM_GUI_ACTIVE / 8 XCDs; MFMA busy = "
                "SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x kernel cycles); executed "
                "MFMA FLOP = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; LDS conflict rate = "
                "SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; L2 hit = TCC_HIT / (TCC_HIT + "
                "TCC_MISS); clock = kernel cycles / dispatch duration (the clock "
                "the chip held during the kernel).\n\n| kernel | kernel cycles | "
                "clock | MFMA busy | executed MFMA "
                "GFLOP | algorithmic GFLOP | LDS bank-conflict cycles / LDS active | "
                "L2 hit |\n|---|---|---|---|---|---|---|---|\n")
        for k in sorted(vals):
            v = {c: float(np.mean(x)) for c, x in vals[k].items()}
            cyc = v.get("GRBM_GUI_ACTIVE", float("nan")) / n_xcd
            busy = v.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan")) / (n_simd * cyc)
            mops = v.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", float("nan")) * 512 / 1e9
            lds = (v.get("SQ_LDS_BANK_CONFLICT", float("nan")) /
                   max(v.get("SQ_LDS_IDX_ACTIVE", float("nan")), 1.0))
            hit = v.get("TCC_HIT_sum", float("nan"))
            miss = v.get("TCC_MISS_sum", float("nan"))
            ghz = cyc / v["_ns"] if "_ns" in v else float("nan")
            f.write(f"| {k} | {cyc:.0f} | {ghz:.2f} GHz | {busy:.1%} | {mops:.1f} | "
                    f"{alg.get(k, 0) / 1e9:.1f} | {lds:.3f} | "
                    f"{hit / (hit + miss):.1%} |\n")
    print(open(md).read())
    return 0


def sweep(dev) -> int:
    """Forward and the dK/dV and dQ backward stages over N = 1K..32K
    with B*H*N = 2^18 tokens (seeded N(0,1) bf16 inputs), HIP events on the
    launch stream, median of 5 runs of 10 launches; prints a markdown
    table of algorithmic TFLOP/s and the fraction of the 2.5 PF bf16 peak."""
    import torch
    import io_aware_tiled_amd as fa
    stream = torch.cuda.current_stream(dev)

    def timed(fn, reps=10):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / reps)
        return sorted(ts)[2]

    print("| d | causal | B x H x N | forward ms | forward TFLOP/s | % of peak "
          "| dK/dV ms | dQ ms | backward TFLOP/s | % of peak |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    tokens = 1 << 18
    for d in (64, 128):
        for causal in (True, False):
            for N in (1024, 2048, 4096, 8192, 16384, 32768):
                bh = tokens // N
                B, H = (bh // 16, 16) if bh >= 16 else (1, bh)
                g = torch.Generator(device=dev).manual_seed(N + d)
                q, k, v, do = (torch.randn(B, H, N, d, device=dev, generator=g)
                               .to(torch.bfloat16) for _ in range(4))
                o = torch.empty_like(q)
                lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
                sc = 1.0 / math.sqrt(d)
                pairs = B * H * (N * (N + 1) // 2 if causal else N * N)
                tf = timed(lambda: fa.fa_fwd(q, k, v, o, lse, sc, causal))
                row = (f"| {d} | {causal} | {B} x {H} x {N} | {tf:.3f} | "
                       f"{4 * d * pairs / tf / 1e9:.0f} | "
                       f"{4 * d * pairs / tf / 1e9 / PEAK_BF16_TFLOPS:.1%} |")
                ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d),
                                 dtype=torch.uint8, device=dev)
                dq, dk, dv = (torch.empty_like(q) for _ in range(3))
                fa.fa_bwd_preprocess(o, do, ws)
                tk = timed(lambda: fa.fa_bwd_dkdv(q, k, v, do, lse, dk, dv, ws,
                                                  sc, causal))
                tq = timed(lambda: fa.fa_bwd_dq(q, k, v, do, lse, dq, ws, sc,
                                                causal))
                tb = 10 * d * pairs / (tk + tq) / 1e9
                row += (f" {tk:.3f} | {tq:.3f} | {tb:.0f} | "
                        f"{tb / PEAK_BF16_TFLOPS:.1%} |")
                print(row, flush=True)
                del q, k, v, do, o, lse, ws, dq, dk, dv
    return 0


def mfma_ceiling(dev, n: int = 8192, iters: int = 20) -> dict:
    """Sustained bf16 matrix-core rate of a vendor GEMM (torch.matmul, n^3)
    on iid N(0,1) operands and on constant operands.  The chip's clock under
    matrix-core load depends on how much the operand bits toggle, so the
    random-operand rate, not the published peak, is what a kernel on real
    data can reach; the constant-operand rate shows the published peak's
    clock."""
    import torch
    g = torch.Generator(device=dev).manual_seed(0)
    out = {"gemm": f"torch.matmul bf16 {n}x{n}x{n}", "iters": iters}
    for kind in ("random", "constant"):
        if kind == "random":
            a = torch.randn(n, n, generator=g, device=dev).to(torch.bfloat16)
            b = torch.randn(n, n, generator=g, device=dev).to(torch.bfloat16)
        else:
            a = torch.full((n, n), 1.0, device=dev, dtype=torch.bfloat16)
            b = torch.full((n, n), 1.0 / 1024, device=dev, dtype=torch.bfloat16)
        c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
        for _ in range(3):
            torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
        e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
        e0.record()
        for _ in range(iters):
            torch.matmul(a, b, out=c)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        out[f"{kind}_tflops"] = round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1)
        del a, b, c
    return out


def summarize_ceiling(path, command) -> int:
    """profiles/mfma_ceiling.md from a rocprofv3 --pmc GRBM_GUI_ACTIVE
    SQ_VALU_MFMA_BUSY_CYCLES collection of a --ceiling-only run: duration,
    held clock and matrix-core busy of the GEMM dispatches, random operands
    (the first half, in dispatch order) versus constant ones."""
    import csv
    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            d = per.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"]})
            d[r["Counter_Name"]] = float(r["Counter_Value"])
            d["ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    total = {}
    for d in per.values():
        total[d["name"]] = total.get(d["name"], 0.0) + d["ns"]
    gemm = max(total, key=total.get)
    ids = sorted(i for i, d in per.items() if d["name"] == gemm)
    half = len(ids) // 2
    n = 8192
    md = os.path.join(PROFILES, "mfma_ceiling.md")
    with open(md, "w") as f:
        f.write("# Matrix-core rate a kernel can sustain on real data\n\n"
                "Command (repository root, one MI355X):\n\n```\n"
                f"{command}\n```\n\nThe vendor bf16 GEMM (torch.matmul, "
                f"{n}^3, {len(ids)} dispatches of `{gemm[:60]}`) first on iid "
                "N(0,1) operands, then on constant operands.  Clock = "
                "GRBM_GUI_ACTIVE / 8 XCDs / dispatch duration; MFMA busy = "
                "SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles).\n\n"
                "| operands | dispatches | mean duration | TFLOP/s | clock | "
                "MFMA busy |\n|---|---|---|---|---|---|\n")
        for label, sel in (("iid N(0,1)", ids[:half]), ("constant", ids[half:])):
            ns = float(np.mean([per[i]["ns"] for i in sel]))
            cyc = float(np.mean([per[i]["GRBM_GUI_ACTIVE"] for i in sel])) / 8
            busy = float(np.mean([per[i]["SQ_VALU_MFMA_BUSY_CYCLES"]
                                  for i in sel])) / (1024 * cyc)
            f.write(f"| {label} | {len(sel)} | {ns / 1e3:.1f} us | "
                    f"{2.0 * n ** 3 / ns / 1e3:.0f} | {cyc / ns:.2f} GHz | "
                    f"{busy:.1%} |\n")
    print(open(md).read())
    return 0


def summarize_trace(w: S.Workload, path, command) -> int:
    import csv
    with open(path) as f:
        rows = [r for r in csv.DictReader(f) if "fa::" in r["Name"]]
    md = os.path.join(PROFILES, f"kernels_{w.name}.md")
    with open(md, "w") as f:
        f.write(f"# Kernel trace: {w.name} (B={w.B} H={w.H} N={w.N} d={w.d}, "
                f"causal={w.causal}, {'forward+backward' if w.backward else 'forward'})"
                f"\n\nCommand (repository root, one MI355X):\n\n```\n{command}"
                "\n```\n\nrocprofv3 kernel statistics, libfa kernels only "
                "(durations in microseconds):\n\n| kernel | calls | average | "
                "min | max | share of GPU time |\n|---|---|---|---|---|---|\n")
        for r in rows:
            name = (r["Name"].replace("(anonymous namespace)::", "")
                    .split("(")[0].replace("void ", ""))
            f.write(f"| `{name}` | {r['Calls']} | {float(r['AverageNs'])/1e3:.1f}"
                    f" | {float(r['MinNs'])/1e3:.1f} | {float(r['MaxNs'])/1e3:.1f}"
                    f" | {float(r['Percentage']):.1f}% |\n")
    print(open(md).read())
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    choices=sorted(S.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (profiling runs)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run an elementwise copy (y = -x, float32) of "
                         "MIB MiB three times after the warmup: the known-size "
                         "kernel that scales rocprofv3 FETCH_SIZE/WRITE_SIZE")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: turn two rocprofv3 --pmc counter "
                         "collections (FETCH_SIZE, then WRITE_SIZE) of a "
                         "--copy-calibration run into profiles/traffic.json "
                         "(give the same --copy-calibration MIB)")
    ap.add_argument("--summarize-trace", metavar="KERNEL_STATS_CSV",
                    help="no GPU work: write the libfa rows of a rocprofv3 "
                         "--kernel-trace --stats kernel_stats.csv to "
                         "profiles/kernels_<workload>.md")
    ap.add_argument("--summarize-counters", nargs=2,
                    metavar=("SQ_CSV", "TCC_CSV"),
                    help="no GPU work: turn two rocprofv3 --pmc collections "
                         "(SQ/GRBM counters, then TCC_HIT_sum TCC_MISS_sum) "
                         "into profiles/counters_<workload>.md")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the vendor-GEMM matrix-core calibration")
    ap.add_argument("--ceiling-only", action="store_true",
                    help="run only the vendor-GEMM calibration (random, then "
                         "constant operands) and print it")
    ap.add_argument("--summarize-ceiling", metavar="PMC_CSV",
                    help="no GPU work: write profiles/mfma_ceiling.md from a "
                         "rocprofv3 --pmc GRBM_GUI_ACTIVE "
                         "SQ_VALU_MFMA_BUSY_CYCLES run of --ceiling-only")
    ap.add_argument("--sweep", action="store_true",
                    help="time the bf16 forward and backward kernels over "
                         "sequence lengths 1K..32K at a fixed token count "
                         "and print a markdown table")
    ap.add_argument("--command", default="",
                    help="with --traffic-from / --summarize-trace: the "
                         "command that made the CSVs")
    args = ap.parse_args(argv)

    if args.summarize_ceiling:
        return summarize_ceiling(args.summarize_ceiling, args.command)
    if args.summarize_counters:
        return summarize_counters(S.WORKLOADS[args.workload],
                                  args.summarize_counters, args.command)
    if args.summarize_trace:
        return summarize_trace(S.WORKLOADS[args.workload], args.summarize_trace,
                               args.command)
    if args.traffic_from:
        if not args.copy_calibration:
            ap.error("--traffic-from needs the run's --copy-calibration MIB")
        return write_traffic(S.WORKLOADS[args.workload], args.traffic_from,
                             args.command, args.copy_calibration)

    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU "
              f"path (asked for --gpus {args.gpus}); run with --gpus 1.",
              file=sys.stderr)
        return 2

    import torch
    import io_aware_tiled_amd as fa

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    if args.ceiling_only:
        print(json.dumps(mfma_ceiling(dev)), flush=True)
        return 0
    if args.sweep:
        return sweep(dev)
    w = S.WORKLOADS[args.workload]
    log(f"[bench] generating {w.name} inputs")
    inp = S.make_inputs(w)

    def up(name):
        bits = inp[name + "_bits"]
        if w.dtype == "bf16":
            return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(bits).to(dev)

    q, k, v = up("q"), up("k"), up("v")
    do = up("do") if w.backward else None
    kv = None if inp["kv_len"] is None else torch.from_numpy(inp["kv_len"]).to(dev)
    bmask = (None if inp.get("block_mask") is None
             else torch.from_numpy(inp["block_mask"]).to(dev))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    scale, causal = inp["scale"], inp["causal"]
    fp8 = inp.get("signs") is not None
    dr = inp.get("dropout")
    if w.linear:
        nl = fa.fa_linear_workspace_size(w.B, w.H, w.N, w.d)
        wsl = torch.empty(nl, dtype=torch.uint8, device=dev) if nl else None
    if fp8:
        signs = torch.from_numpy(inp["signs"]).to(dev)
        ws8 = torch.empty(fa.fa_fp8_workspace_size(w.B, w.H, w.N, w.d),
                          dtype=torch.uint8, device=dev)
        score_scale = float(np.float32(scale) / np.float32(w.d))
    if w.backward:
        ws = torch.empty(fa.fa_bwd_workspace_size(w.B, w.H, w.N, w.d),
                         dtype=torch.uint8, device=dev)
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    names = ["fwd"] + (["bwd_preprocess", "bwd_dkdv", "bwd_dq"]
                       if w.backward else [])
    if fp8:
        names = ["fp8_quantize", "fwd_fp8"]
    if w.linear:
        names = ["linear_fwd"]

    def step(events=None):
        def mark(i):
            if events is not None:
                events[i].record(stream)
        mark(0)
        if w.linear:
            fa.fa_linear_fwd(q, k, v, o, scale, wsl)
            mark(1)
            return
        if fp8:
            fa.fa_fp8_quantize(q, k, v, signs, ws8)
            mark(1)
            fa.fa_fwd_fp8_quantized(ws8, o, lse, score_scale, causal)
            mark(2)
            return
        if w.dtype == "f32":
            fa.fa_fwd_f32(q, k, v, o, lse, scale, causal)
        elif dr is not None:
            fa.fa_fwd_dropout(q, k, v, o, lse, scale, causal, dr["p"],
                              dr["seed"], dr["offset"])
        elif bmask is not None:
            fa.fa_fwd_block_sparse(q, k, v, bmask, o, lse, scale, causal)
        else:
            fa.fa_fwd_kvlen(q, k, v, kv, o, lse, scale, causal)
        mark(1)
        if w.backward:
            fa.fa_bwd_preprocess(o, do, ws)
            mark(2)
            if dr is not None:
                fa.fa_bwd_dkdv_dropout(q, k, v, do, lse, dk, dv, ws, scale,
                                       causal, dr["p"], dr["seed"], dr["offset"])
            elif bmask is not None:
                fa.fa_bwd_dkdv_block_sparse(q, k, v, do, lse, bmask, dk, dv,
                                            ws, scale, causal)
            else:
                fa.fa_bwd_dkdv(q, k, v, do, lse, dk, dv, ws, scale, causal)
            mark(3)
            if dr is not None:
                fa.fa_bwd_dq_dropout(q, k, v, do, lse, dq, ws, scale, causal,
                                     dr["p"], dr["seed"], dr["offset"])
            elif bmask is not None:
                fa.fa_bwd_dq_block_sparse(q, k, v, do, lse, bmask, dq, ws,
                                          scale, causal)
            else:
                fa.fa_bwd_dq(q, k, v, do, lse, dq, ws, scale, causal)
            mark(4)

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        cx = torch.ones(n, dtype=torch.float32, device=dev)
        cy = torch.empty_like(cx)
        for _ in range(3):
            torch.neg(cx, out=cy)
        torch.cuda.synchronize()
        del cx, cy
        log(f"[bench] copy calibration: 3 x {args.copy_calibration} MiB")

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
          for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps

    per_kernel = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in ev]))
                  for j, n in enumerate(names)}
    pairs = visible_pairs(w, inp["kv_len"], inp.get("block_mask"))
    fwd_flops = linear_flops(w) if w.linear else 4.0 * w.d * pairs
    bwd_flops = 10.0 * w.d * pairs if w.backward else 0.0
    step_flops = fwd_flops + bwd_flops
    value = step_flops / (ms_step * 1e-3) / 1e12
    peak = (PEAK_F32_TFLOPS if w.dtype == "f32" else
            PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS)

    if w.backward:
        # fa_bwd_dkdv produces dK and dV: S = Q K^T, dP = dO V^T, dV += P^T dO
        # and dK += dS^T Q, 2d FLOP each per visible pair.
        dom, dom_flops, src = ("bwd_dkdv", 8.0 * w.d * pairs,
                               ["fa_bwd.hip", "fa_common.h"])
    elif w.linear:
        dom, dom_flops, src = ("linear_fwd", fwd_flops,
                               ["fa_linear.hip", "fa_common.h"])
    elif fp8:
        # the attention kernel on the quantised operands (the quantisation
        # pass is HBM-bound and reported in kernel_ms)
        dom, dom_flops, src = ("fwd_fp8", fwd_flops,
                               ["fa_fp8.hip", "fa_common.h"])
    else:
        dom, dom_flops, src = "fwd", fwd_flops, ["fa_fwd.hip", "fa_common.h"]
    dom_ms = per_kernel[dom]
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        ent = tr.get(w.name, {}).get("kernels", {}).get(dom)
        if ent and ent.get("source_digest") == _sources_digest(src):
            traffic = ent["bytes_per_launch"]
    roofline = {"bound": "mfma", "achieved": round(achieved, 2),
                "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic,
                "kernel": dom, "kernel_ms": round(dom_ms, 4),
                "algorithmic_flop_per_launch": dom_flops}
    if w.linear:
        # ~80 FLOP per compulsory byte at d = 128: HBM, not the matrix
        # cores, bounds it.
        nbytes = algorithmic_bytes(w, dom)
        gbs = nbytes / (dom_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 1),
                    "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                    "kernel": dom, "kernel_ms": round(dom_ms, 4),
                    "algorithmic_bytes_per_launch": nbytes,
                    "algorithmic_flop_per_launch": dom_flops}

    # outputs of the timed run must be finite (parity itself is the tests' job)
    check = {"o_finite": bool(torch.isfinite(o.float()).all()),
             "lse_finite_or_neg_inf": bool((torch.isfinite(lse) | (lse == -float("inf"))).all())}
    if w.backward:
        check["grads_finite"] = bool(all(torch.isfinite(t.float()).all()
                                         for t in (dq, dk, dv)))

    ceiling = None
    if not args.no_ceiling and w.dtype == "bf16" and not fp8 and not w.linear:
        log("[bench] vendor GEMM calibration of the matrix-core rate")
        ceiling = mfma_ceiling(dev)
        ceiling["frac_of_random"] = round(achieved / ceiling["random_tflops"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on a sample (cpu_baseline)")
        cpu = cpu_baseline(w, inp)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "f32" if w.dtype == "f32" else "fp8_e4m3" if fp8 else "bf16",
        "data": "synthetic (seeded iid N(0,1) inputs of the workload's shape)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal,
                   "pass": ("forward+backward" if w.backward else
                            "linear attention forward" if w.linear else "forward"),
                   "parallelism": "single GPU"},
        "frac_of_peak": round(value / peak, 4),
        "kernel_ms": {n: round(t, 4) for n, t in per_kernel.items()},
        "fwd_tflops": round(fwd_flops / (per_kernel[dom if (fp8 or w.linear)
                                                    else "fwd"]
                                         * 1e-3) / 1e12, 2),
        "roofline": roofline,
        "mfma_ceiling": ceiling,
        "cpu_baseline": cpu,
        "sanity": check,
    }
    if dr is not None:
        out["dropout"] = {"p": dr["p"], "seed": dr["seed"],
                          "offset": dr["offset"],
                          "generator": "Philox4x32-10, one byte per pair",
                          "flops": "algorithmic (generator work not counted)"}
    if fp8:
        qb = algorithmic_bytes(w, "fp8_quantize")
        out["fp8"] = {
            "quantize_ms": round(per_kernel["fp8_quantize"], 4),
            "quantize_algorithmic_bytes": qb,
            "quantize_gb_per_s": round(qb / (per_kernel["fp8_quantize"] * 1e-3) / 1e9, 1),
            "rotation": "randomised Hadamard (seeded signs)",
            "blocks": "32 values, E8M0 scale; E4M3 codes"}
        out["data"] = ("synthetic (seeded iid N(0,1) bf16 inputs of the "
                       "workload's shape, quantised on the GPU each step)")
    if w.backward:
        bwd_ms = sum(per_kernel[n] for n in names[1:])
        out["bwd_tflops"] = round(bwd_flops / (bwd_ms * 1e-3) / 1e12, 2)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
