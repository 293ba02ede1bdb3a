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
sample of heads on the host cores).  A "steady_state" object repeats the
timing after --steady-s more seconds of untimed steps: a GPU that was idle
while the inputs were generated runs its first steps at a lower clock, so
that object gives the rate under sustained load beside the contract's one.
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
            if w.backward:
                oracle.linear.linear_attention_bwd(q, k, v, inp["do"][sl],
                                                   inp["scale"])
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
        sw = S.Workload(w.name, 1, nh, w.N, w.d, w.dtype, True, w.seeds,
                        w.backward, linear=True)
        flops = linear_flops(sw) + (linear_bwd_flops(sw) if w.backward else 0)
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
        what = ("fp64 numpy causal linear attention (quadratic definition"
                + (", analytic gradients)" if w.backward else ")"))
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


def linear_bwd_flops(w: S.Workload) -> float:
    """Algorithmic FLOPs of the chunkwise linear-attention backward: per
    visible pair inside a chunk 4d for each of dQ, dK and dV (a score and
    its product); per row 4d^2 for dQ's state (update and use) and 6d^2
    for dK and dV (one shared state, which the kernels build twice, and
    its two uses)."""
    full, rem = divmod(w.N, LINEAR_CHUNK)
    intra = full * LINEAR_CHUNK * (LINEAR_CHUNK + 1) // 2 + rem * (rem + 1) // 2
    return w.B * w.H * (12.0 * w.d * intra + 10.0 * w.N * w.d * w.d)


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
    if kernel == "linear_bwd":                   # Q,K,V,dO -> dQ,dK,dV
        return 7 * t
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


# The pages' own figures for exact tiled attention against the standard
# (score-materialising) implementation, quoted as context: what they time
# and on which hardware is the pages' (no hardware is named for these).
PAGE_FIGURES = (
    {"figure": "15% faster", "workload": "BERT-large, sequence length 512",
     "hardware": "not stated",
     "source": "Paper summary: FlashAttention (zenn.dev), Overview"},
    {"figure": "3x faster", "workload": "GPT-2, sequence length 1K",
     "hardware": "not stated",
     "source": "Paper summary: FlashAttention (zenn.dev), Overview"},
    {"figure": "2.4x faster", "workload": "Long Range Arena, sequence length 1K-4K",
     "hardware": "not stated",
     "source": "Paper summary: FlashAttention (zenn.dev), Overview"},
    {"figure": "about 20x less memory", "workload": "against standard attention",
     "hardware": "not stated",
     "source": "Paper summary: FlashAttention (zenn.dev), Experimental results"},
    {"figure": "about 12.9 GB of fp16 scores", "workload": "12 heads, N = 23,400",
     "hardware": "-",
     "source": "Is a full-day context better than a 10-minute context? (marketmaker.cc), introduction"},
)
CONTEXT_WORKLOADS = ("gpt2_causal", "bert_keypad", "tradingday_causal")


def standard_attention(q, k, v, scale: float, causal: bool, kv_len):
    """The standard attention the pages compare against: S = scale Q K^T
    written out (in the inputs' dtype, bf16 here), masked, softmax in fp32,
    P written out in the inputs' dtype, O = P V.  Measurement only (timing
    and memory beside fa_fwd)."""
    import torch
    s = torch.matmul(q, k.transpose(-1, -2).contiguous())
    s.mul_(scale)
    n = q.shape[2]
    if causal:
        s.masked_fill_(torch.ones(n, n, dtype=torch.bool, device=q.device).triu_(1),
                       float("-inf"))
    if kv_len is not None:
        keys = torch.arange(n, device=q.device)
        s.masked_fill_((keys[None, :] >= kv_len[:, None].long())[:, None, None, :],
                       float("-inf"))
    p = torch.softmax(s, dim=-1, dtype=torch.float32).to(q.dtype)
    del s
    return torch.matmul(p, v)


def context_vs_standard(dev) -> dict:
    """The pages' figures (PAGE_FIGURES) beside the same comparison made
    here: fa_fwd against standard_attention on the GPT-2, BERT and
    trading-day shapes, time (median of 5 timings) and device memory
    beyond the inputs (the standard path's peak, fa_fwd's O and LSE: the
    library allocates nothing)."""
    import torch
    import io_aware_tiled_amd as fa
    out = {"pages": list(PAGE_FIGURES), "measured_here": {}}

    def med_ms(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / reps)
        return sorted(ts)[2]

    for name in CONTEXT_WORKLOADS:
        w = S.WORKLOADS[name]
        log(f"[bench] context: {name} against standard attention")
        inp = S.make_inputs(w)
        up = lambda n: torch.from_numpy(inp[n + "_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
        q, k, v = up("q"), up("k"), up("v")
        kv = None if inp["kv_len"] is None else torch.from_numpy(inp["kv_len"]).to(dev)
        scale, causal = inp["scale"], inp["causal"]
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        fa_extra = o.numel() * o.element_size() + lse.numel() * lse.element_size()
        fa_ms = med_ms(lambda: fa.fa_fwd_kvlen(q, k, v, kv, o, lse, scale, causal), 20)
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats(dev)
        m1 = torch.cuda.memory_allocated(dev)
        o_std = standard_attention(q, k, v, scale, causal, kv)
        torch.cuda.synchronize()
        std_extra = torch.cuda.max_memory_allocated(dev) - m1
        diff = float((o_std.float() - o.float()).abs().max())
        del o_std
        reps = 2 if w.N > 8192 else 20
        std_ms = med_ms(lambda: standard_attention(q, k, v, scale, causal, kv), reps)
        out["measured_here"][name] = {
            "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
            "standard_ms": round(std_ms, 4), "fa_fwd_ms": round(fa_ms, 4),
            "speedup": round(std_ms / fa_ms, 2),
            "standard_extra_bytes": int(std_extra),
            "fa_fwd_extra_bytes": int(fa_extra),
            "memory_ratio": round(std_extra / fa_extra, 1),
            "bf16_scores_bytes": int(w.B * w.H * w.N * w.N * 2),
            "max_abs_diff_o": diff}
        del q, k, v, kv, o, lse
        torch.cuda.empty_cache()
    out["what"] = ("forward only, one GPU; standard = S and P written to HBM "
                   "(bf16), fp32 softmax, vendor GEMMs; fa_fwd = this library")
    return out


STALL_COUNTERS = (
    ("SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY "
     "SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS "
     "SQ_ACTIVE_INST_SCA GRBM_GUI_ACTIVE"),
    ("SQ_WAIT_INST_LDS SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_SALU "
     "SQ_INSTS_VALU_TRANS_F32 SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_MISC "
     "GRBM_GUI_ACTIVE"))


def _pmc_means(csvs) -> dict:
    """{kernel key: {counter: mean over dispatches}} of rocprofv3 --pmc
    counter_collection CSVs (libfa kernels only)."""
    import csv
    vals = {}
    for path in csvs:
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
    return {k: {c: float(np.mean(x)) for c, x in d.items()} for k, d in vals.items()}


def summarize_stalls(w: S.Workload, csvs, command) -> int:
    """profiles/stalls_<workload>.md: where the wavefronts' cycles go (SQ
    wave-cycle counters as fractions of SQ_WAVE_CYCLES, the same units) and
    the instruction mix per MFMA, from two rocprofv3 --pmc collections
    (STALL_COUNTERS) of a bench run."""
    v = _pmc_means(csvs)
    md = os.path.join(PROFILES, f"stalls_{w.name}.md")
    frac = (("SQ_ACTIVE_INST_ANY", "issuing any"), ("SQ_ACTIVE_INST_VALU", "VALU"),
            ("SQ_ACTIVE_INST_LDS", "LDS"), ("SQ_ACTIVE_INST_SCA", "scalar"),
            ("SQ_ACTIVE_INST_MISC", "misc"), ("SQ_WAIT_INST_ANY", "waiting to issue"),
            ("SQ_WAIT_INST_LDS", "waiting on LDS issue"), ("SQ_WAIT_ANY", "waiting (any)"))
    with open(md, "w") as f:
        f.write(f"# Where the cycles go: {w.name} (B={w.B} H={w.H} N={w.N} d={w.d}, "
                f"causal={w.causal})\n\nCommands (repository root, one MI355X):"
                f"\n\n```\n{command}\n```\n\nPer dispatch (mean over the run's "
                "dispatches).  The SQ wave-cycle counters are given as fractions "
                "of SQ_WAVE_CYCLES (summed over wavefronts, same units); a "
                "wavefront can be issuing one kind of instruction while waiting "
                "on another, so the fractions do not add up to one.  MFMA busy = "
                "SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8).  "
                "Instruction counts are per MFMA instruction (SQ_INSTS_*; "
                "transcendental = SQ_INSTS_VALU_TRANS_F32).\n\n")
        f.write("| kernel | MFMA busy | " + " | ".join(n for _, n in frac) +
                " | VALU / MFMA | transc. / MFMA | LDS / MFMA | SALU / MFMA |\n")
        f.write("|---" * (6 + len(frac)) + "|\n")
        for k in sorted(v):
            c = v[k]
            wc = c.get("SQ_WAVE_CYCLES", float("nan"))
            cyc = c.get("GRBM_GUI_ACTIVE", float("nan")) / 8
            busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan")) / (1024 * cyc)
            # (SQ_INSTS_VALU counts the MFMA instructions too)
            nm = c.get("SQ_INSTS_MFMA", float("nan"))
            cells = [f"{busy:.1%}"] + [f"{c.get(n, float('nan')) / wc:.3f}"
                                       for n, _ in frac]
            cells += [f"{c.get(n, float('nan')) / nm:.2f}" if nm else "—" for n in (
                "SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_LDS",
                "SQ_INSTS_SALU")]
            f.write(f"| {k} | " + " | ".join(cells) + " |\n")
    print(open(md).read())
    return 0


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


def summarize_trace(w: S.Workload, path, command, warmup: int,
                    steps: int, steady_warm: int = -1) -> int:
    """profiles/kernels_<workload>.md from a rocprofv3 kernel trace: per
    libfa kernel, the timed dispatches only.  The run made T = warmup +
    steps steps, or, when it made a steady-state pass of steady_warm
    untimed steps and `steps` timed ones (bench.py logs the count), T =
    warmup + 2 steps + steady_warm.  A kernel that each step runs c times
    (c T dispatches) has its first c warmup dispatches skipped and the next
    c steps kept; with a steady-state pass its last c steps are reported
    beside them."""
    import csv
    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if "fa::" not in r["Kernel_Name"]:
                continue
            ns = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            per.setdefault(r["Kernel_Name"], []).append(
                (int(r["Dispatch_Id"]), ns))
    md = os.path.join(PROFILES, f"kernels_{w.name}.md")
    steady = steady_warm >= 0
    n_run = warmup + steps + (steps + steady_warm if steady else 0)
    for name, v in per.items():
        if len(v) % n_run:
            raise SystemExit(f"{name}: {len(v)} dispatches, not a multiple of "
                             f"the run's {n_run} steps")
    with open(md, "w") as f:
        f.write(f"# Kernel trace: {w.name} (B={w.B} H={w.H} N={w.N} d={w.d}, "
                f"causal={w.causal}, {'forward+backward' if w.backward else 'forward'})"
                f"\n\nCommand (repository root, one MI355X):\n\n```\n{command}"
                "\n```\n\nrocprofv3 kernel trace, libfa kernels only, the "
                f"timed dispatches of each kernel (the dispatches of its first "
                f"{warmup} steps are the warmup and are skipped, those of the "
                f"next {steps} are kept; durations in microseconds)")
        if steady:
            f.write(f", and beside them the last {steps} steps of the run "
                    f"(the steady-state pass: {steady_warm} more untimed "
                    "steps, then those)")
        f.write(":\n\n| kernel | timed dispatches | average | min | max |"
                + (" steady average | steady min | steady max |" if steady else "")
                + "\n|---|---|---|---|---|" + ("---|---|---|" if steady else "")
                + "\n")
        for name, v in sorted(per.items(), key=lambda kv: -sum(x[1] for x in kv[1])):
            c = len(v) // n_run
            v = sorted(v)
            d = np.array([ns for _, ns in v[c * warmup:c * (warmup + steps)]],
                         dtype=np.float64) / 1e3
            if not len(d):
                continue
            short = (name.replace("(anonymous namespace)::", "")
                     .split("(")[0].replace("void ", ""))
            row = (f"| `{short}` | {len(d)} | {d.mean():.1f} | {d.min():.1f} "
                   f"| {d.max():.1f} |")
            if steady:
                e = np.array([ns for _, ns in v[-c * steps:]], dtype=np.float64) / 1e3
                row += f" {e.mean():.1f} | {e.min():.1f} | {e.max():.1f} |"
            f.write(row + "\n")
    print(open(md).read())
    return 0


MICRO_LIB = os.path.join(ROOT, "microbench", "libmicro.so")


def micro(command: str) -> int:
    """Microbenchmarks of the hardware features the kernels rely on
    (microbench/micro.hip), one workgroup of 256 x wps threads per CU on
    every CU; writes profiles/microbench.md.  Cycles are shader-clock cycles
    per wavefront (s_memtime) over the timed loop; the clock is cycles per
    microsecond of the 100 MHz constant clock (s_memrealtime)."""
    import ctypes
    import torch
    if not os.path.exists(MICRO_LIB):
        print(f"{MICRO_LIB} is missing: build it with "
              "`python -m io_aware_tiled_amd.build`", file=sys.stderr)
        return 1
    torch.cuda.init()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    L = ctypes.CDLL(MICRO_LIB)
    L.micro_run.restype = ctypes.c_int
    L.micro_run.argtypes = [ctypes.c_int] * 5 + [ctypes.POINTER(ctypes.c_double)] * 3

    def run(which, wps, constant, iters):
        c, u, ms = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
        st = L.micro_run(which, wps, constant, iters, cus, ctypes.byref(c),
                         ctypes.byref(u), ctypes.byref(ms))
        if st != 0:
            raise RuntimeError(f"micro_run({which}) failed: HIP error {st}")
        return c.value, u.value, ms.value

    rows = []
    # matrix cores: 4 independent chains (throughput), 1 chain (latency)
    for chains, which in ((4, 1), (1, 0)):
        for constant in (0, 1):
            for wps in (1, 2):
                it = 2000
                c, u, ms = run(which, wps, constant, it)
                n = it * chains
                flop = cus * 4 * wps * n * 32768.0
                rows.append(("v_mfma_f32_32x32x16_bf16", f"{chains} chain(s), "
                             + ("constant" if constant else "random") + " operands",
                             wps, f"{c / n:.1f} cycles/MFMA per wave",
                             f"{flop / (ms * 1e-3) / 1e12:.0f} TFLOP/s, {c / u / 1e3:.2f} GHz"))
    for which, name in ((2, "v_fma_f32"), (4, "v_add_f32"), (9, "v_exp_f32"),
                        (3, "v_exp_f32 + v_fma_f32")):
        for wps in (1, 2, 4):
            it = 4000
            c, u, ms = run(which, wps, 0, it)
            ghz = c / u / 1e3
            # SIMD cycles per instruction over the whole kernel (the waves of
            # a SIMD need not run their loops at the same time)
            simd = ms * 1e-3 * ghz * 1e9 / (it * 8 * wps)
            rows.append((name, "8 independent chains", wps,
                         f"{c / (it * 8):.2f} cycles/instruction per wave, "
                         f"{simd:.2f} SIMD cycles per instruction over the "
                         f"kernel time", f"{ghz:.2f} GHz"))
    for wps in (1, 2):
        it = 2000
        c0, _, ms0 = run(1, wps, 0, it)
        c1, u1, ms1 = run(5, wps, 0, it)
        flop = cus * 4 * wps * it * 4 * 32768.0
        rows.append(("MFMA + 4 FMA after each", "4 MFMA chains, random", wps,
                     f"{c1 / (it * 4):.1f} cycles per MFMA slot per wave (MFMA "
                     f"alone {c0 / (it * 4):.1f})",
                     f"{flop / (ms1 * 1e-3) / 1e12:.0f} TFLOP/s (MFMA alone "
                     f"{flop / (ms0 * 1e-3) / 1e12:.0f}), {c1 / u1 / 1e3:.2f} GHz"))
    for which, name in ((10, "MFMA + 4 SALU after each"),
                        (11, "MFMA + 4 s_nop 0 after each"),
                        (12, "MFMA + 4 s_waitcnt after each"),
                        (13, "MFMA + 4 ds_read_b128 after each"),
                        (14, "MFMA + 1 ds_read_b128 after each"),
                        (15, "MFMA + 2 ds_read_b64_tr_b16 after each"),
                        (16, "MFMA (AGPR acc.) + 1 ds_read_b128 after each"),
                        (17, "MFMA (AGPR acc.) alone")):
        for wps in (1, 2):
            it = 2000
            c0, _, ms0 = run(1, wps, 0, it)
            c1, u1, ms1 = run(which, wps, 0, it)
            flop = cus * 4 * wps * it * 4 * 32768.0
            rows.append((name, "4 MFMA chains, random", wps,
                         f"{c1 / (it * 4):.1f} cycles per MFMA slot per wave (MFMA "
                         f"alone {c0 / (it * 4):.1f})",
                         f"{flop / (ms1 * 1e-3) / 1e12:.0f} TFLOP/s (MFMA alone "
                         f"{flop / (ms0 * 1e-3) / 1e12:.0f}), {c1 / u1 / 1e3:.2f} GHz"))
    for which, name in ((20, "16x16x32 MFMA alone (register operands)"),
                        (21, "16x16x32 MFMA + 1 ds_read_b128 operand each"),
                        (22, "16x16x32 MFMA + 2 ds_read_b64_tr_b16 operand each"),
                        (23, "16x16x32 MFMA + the two alternating")):
        for wps in (1, 2):
            it = 2000
            c1, u1, ms1 = run(which, wps, 0, it)
            flop = cus * 4 * wps * it * 16 * 16384.0
            rows.append((name, "4 chains, operand ring 4 deep, 304-byte rows, random",
                         wps, f"{c1 / (it * 16):.1f} cycles per MFMA per wave",
                         f"{flop / (ms1 * 1e-3) / 1e12:.0f} TFLOP/s, "
                         f"{c1 / u1 / 1e3:.2f} GHz"))
    for which, name in ((24, "32x32x16 MFMA + 1 ds_read_b128 operand each"),
                        (25, "32x32x16 MFMA + 2 ds_read_b64_tr_b16 operand each"),
                        (26, "32x32x16 MFMA + the two alternating")):
        for wps in (1, 2):
            it = 2000
            c1, u1, ms1 = run(which, wps, 0, it)
            flop = cus * 4 * wps * it * 16 * 32768.0
            rows.append((name, "4 chains, operand ring 4 deep, 304-byte rows, random",
                         wps, f"{c1 / (it * 16):.1f} cycles per MFMA per wave",
                         f"{flop / (ms1 * 1e-3) / 1e12:.0f} TFLOP/s, "
                         f"{c1 / u1 / 1e3:.2f} GHz"))
    for which, name, per, rowb in ((6, "ds_read_b128 (row slices)", 1024, 272),
                                   (7, "2 x ds_read_b64_tr_b16 (transposed)", 1024, 320),
                                   (18, "ds_read_b128 (row slices)", 1024, 304),
                                   (19, "2 x ds_read_b64_tr_b16 (transposed)", 1024, 304)):
        for wps in (1, 2, 4):
            it = 4000
            c, u, ms = run(which, wps, 0, it)
            byts = 4 * wps * it * 8 * per
            ghz = c / u / 1e3
            agg = byts / (ms * 1e-3 * ghz * 1e9)   # per CU over the kernel time
            rows.append((name, f"8 operands per iteration, {rowb}-byte rows", wps,
                         f"{byts / c:.0f} bytes/cycle per CU (per-wave loop "
                         f"time), {agg:.0f} over the kernel time",
                         f"{ghz:.2f} GHz"))
    for wps in (1, 2, 4):
        it = 2000
        c, u, _ = run(8, wps, 0, it)
        byts = 4 * wps * it * 8 * 1024
        rows.append(("buffer_load_dwordx4 ... lds (LDS DMA)",
                     "8 x 1 KB per wave, L2-resident source", wps,
                     f"{byts / c:.0f} bytes/cycle per CU",
                     f"{byts / (c / (c / u)) / 1e3 * cus:.0f} GB/s chip"))
    md = os.path.join(PROFILES, "microbench.md")
    with open(md, "w") as f:
        f.write("# Microbenchmarks (microbench/micro.hip), one MI355X\n\n"
                f"Command (repository root):\n\n```\n{command}\n```\n\n"
                f"One workgroup of 256 x wps threads per CU on all {cus} CUs; "
                "per-wavefront shader cycles (s_memtime) of the timed loop; "
                "clock = cycles / microseconds of s_memrealtime (100 MHz).\n\n"
                "| instruction | pattern | waves per SIMD | result | rate / clock |\n"
                "|---|---|---|---|---|\n")
        for r in rows:
            f.write("| " + " | ".join(str(x) for x in r) + " |\n")
    print(open(md).read(), flush=True)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    choices=sorted(S.WORKLOADS))
    ap.add_argument("--steady-s", type=float, default=0.3, metavar="SECONDS",
                    help="after the timed steps, step untimed for this long "
                         "and time the steps again (steady_state; 0: skip)")
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
    ap.add_argument("--summarize-trace", metavar="KERNEL_TRACE_CSV",
                    help="no GPU work: write the libfa dispatches of a "
                         "rocprofv3 --kernel-trace kernel_trace.csv to "
                         "profiles/kernels_<workload>.md, skipping each "
                         "kernel's first --warmup dispatches and keeping the "
                         "next --steps (the timed ones)")
    ap.add_argument("--steady-warm", type=int, default=-1, metavar="N",
                    help="with --summarize-trace: the traced run made a "
                         "steady-state pass of N untimed steps (its log "
                         "gives N); -1: it made none")
    ap.add_argument("--summarize-counters", nargs=2,
                    metavar=("SQ_CSV", "TCC_CSV"),
                    help="no GPU work: turn two rocprofv3 --pmc collections "
                         "(SQ/GRBM counters, then TCC_HIT_sum TCC_MISS_sum) "
                         "into profiles/counters_<workload>.md")
    ap.add_argument("--summarize-stalls", nargs=2, metavar=("PMC1_CSV", "PMC2_CSV"),
                    help="no GPU work: turn two rocprofv3 --pmc collections "
                         "(the two counter sets of STALL_COUNTERS) into "
                         "profiles/stalls_<workload>.md")
    ap.add_argument("--no-per-config", dest="per_config", action="store_false",
                    help="skip the per-config table (the five synthetic "
                         "configs, each timed and beside its oracle time)")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the comparison with standard attention that "
                         "sits beside the pages' own figures")
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
    ap.add_argument("--micro", action="store_true",
                    help="run the hardware microbenchmarks (microbench/) and "
                         "write profiles/microbench.md")
    ap.add_argument("--command", default="",
                    help="with --traffic-from / --summarize-trace: the "
                         "command that made the CSVs")
    args = ap.parse_args(argv)

    if args.summarize_ceiling:
        return summarize_ceiling(args.summarize_ceiling, args.command)
    if args.summarize_stalls:
        return summarize_stalls(S.WORKLOADS[args.workload],
                                args.summarize_stalls, args.command)
    if args.summarize_counters:
        return summarize_counters(S.WORKLOADS[args.workload],
                                  args.summarize_counters, args.command)
    if args.summarize_trace:
        return summarize_trace(S.WORKLOADS[args.workload], args.summarize_trace,
                               args.command, args.warmup, args.steps,
                               args.steady_warm)
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
    if args.micro:
        return micro(args.command or "python bench.py --micro")
    w = S.WORKLOADS[args.workload]
    res = time_workload(w, dev, args.steps, args.warmup,
                        copy_calibration=args.copy_calibration,
                        steady_s=args.steady_s)
    out = result_line(w, res, args)
    if args.per_config and w.name == DEFAULT_WORKLOAD:
        out["per_config"] = per_config(dev, args, res, out)
        if not args.no_context:
            out["context"] = context_vs_standard(dev)
    print(json.dumps(out), flush=True)
    return 0


# The five synthetic workloads quoted by the metric: (config number, name).
CONFIGS = ((1, "tiny_f32"), (2, "gpt2_causal"), (3, "bert_keypad"),
           (4, "tradingday_causal"), (5, "causal_fwd_bwd_d128"))


def time_workload(w: S.Workload, dev, steps: int, warmup: int,
                  copy_calibration: int = 0, steady_s: float = 0.0,
                  bare_wall: bool = False) -> dict:
    """Upload the workload's inputs, run `warmup` untimed steps, then time
    `steps` steps: wall clock around all of them (synchronised on both
    sides) and HIP events on the launch stream around every kernel.

    With steady_s > 0, after that timed region: keep stepping (untimed) for
    at least steady_s seconds, then time `steps` more steps the same way
    (result["steady"]).  A GPU that has been idle runs its first steps at
    a lower clock, so a few warmup steps after input generation measure
    part of the clock ramp; the second pass gives the sustained rate.

    With bare_wall, the wall clock is taken over `steps` steps that record
    no events and the per-kernel times over `steps` more that do: for
    kernels of a few tens of microseconds the host's event records in each
    step take longer than the kernel, and the wall clock would measure the
    host."""
    import torch
    import io_aware_tiled_amd as fa
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
    dq = dk = dv = None
    if w.backward and w.linear:
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    elif w.backward:
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
        names = ["linear_fwd"] + (["linear_bwd"] if w.backward else [])

    # One zero-argument binding call per kernel, in step order.
    if w.linear:
        stages = [lambda: fa.fa_linear_fwd(q, k, v, o, scale, wsl)]
        if w.backward:
            stages.append(lambda: fa.fa_linear_bwd(q, k, v, do, dq, dk, dv,
                                                   scale, wsl))
    elif fp8:
        stages = [lambda: fa.fa_fp8_quantize(q, k, v, signs, ws8),
                  lambda: fa.fa_fwd_fp8_quantized(ws8, o, lse, score_scale,
                                                  causal)]
    else:
        if w.dtype == "f32":
            fwd = lambda: fa.fa_fwd_f32(q, k, v, o, lse, scale, causal)
        elif dr is not None:
            fwd = lambda: fa.fa_fwd_dropout(q, k, v, o, lse, scale, causal,
                                            dr["p"], dr["seed"], dr["offset"])
        elif bmask is not None:
            fwd = lambda: fa.fa_fwd_block_sparse(q, k, v, bmask, o, lse,
                                                 scale, causal)
        else:
            fwd = lambda: fa.fa_fwd_kvlen(q, k, v, kv, o, lse, scale, causal)
        stages = [fwd]
        if w.backward:
            stages.append(lambda: fa.fa_bwd_preprocess(o, do, ws))
            if dr is not None:
                stages += [
                    lambda: fa.fa_bwd_dkdv_dropout(q, k, v, do, lse, dk, dv, ws,
                                                   scale, causal, dr["p"],
                                                   dr["seed"], dr["offset"]),
                    lambda: fa.fa_bwd_dq_dropout(q, k, v, do, lse, dq, ws, scale,
                                                 causal, dr["p"], dr["seed"],
                                                 dr["offset"])]
            elif bmask is not None:
                stages += [
                    lambda: fa.fa_bwd_dkdv_block_sparse(q, k, v, do, lse, bmask,
                                                        dk, dv, ws, scale,
                                                        causal),
                    lambda: fa.fa_bwd_dq_block_sparse(q, k, v, do, lse, bmask,
                                                      dq, ws, scale, causal)]
            else:
                stages += [
                    lambda: fa.fa_bwd_dkdv(q, k, v, do, lse, dk, dv, ws, scale,
                                           causal),
                    lambda: fa.fa_bwd_dq(q, k, v, do, lse, dq, ws, scale,
                                         causal)]
    assert len(stages) == len(names)
    # Each stage's C calls, marshalled once by the binding (which validates
    # the arguments and turns them into pointers, sizes and the stream); the
    # steps then call the C entry points directly, so a step's host work is
    # a few ctypes calls and event records and short kernels are not left
    # waiting for the host between launches.
    calls = [record_calls(fa, st) for st in stages]

    def step(events=None):
        if events is not None:
            events[0].record(stream)
        for i, cs in enumerate(calls):
            for fn, args in cs:
                st = fn(*args)
                if st != 0:
                    raise fa.FAError(st, names[i])
            if events is not None:
                events[i + 1].record(stream)

    log(f"[bench] {w.name}: warmup {warmup} steps")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    if copy_calibration:
        n = copy_calibration * (1 << 20) // 4
        cx = torch.ones(n, dtype=torch.float32, device=dev)
        cy = torch.empty_like(cx)
        for _ in range(3):
            torch.neg(cx, out=cy)
        torch.cuda.synchronize()
        del cx, cy
        log(f"[bench] copy calibration: 3 x {copy_calibration} MiB")

    def timed():
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
              for _ in range(steps)]
        if bare_wall:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(steps):
                step()
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(ev[i])
        torch.cuda.synchronize()
        if not bare_wall:
            wall = time.perf_counter() - t0
        per_kernel = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in ev]))
                      for j, n in enumerate(names)}
        return per_kernel, wall

    log(f"[bench] {w.name}: timing {steps} steps")
    per_kernel, wall = timed()
    steady = None
    if steady_s > 0:
        # batches of about 20 ms of GPU work between host synchronisations
        batch = max(1, int(20.0 / max(wall * 1e3 / steps, 1e-3)))
        n_warm, t1 = 0, time.perf_counter()
        while time.perf_counter() - t1 < steady_s:
            for _ in range(batch):
                step()
            n_warm += batch
            torch.cuda.synchronize()
        warm_s = time.perf_counter() - t1
        log(f"[bench] {w.name}: {n_warm} more steps ({warm_s:.2f} s), "
            f"timing {steps} steps again")
        pk2, wall2 = timed()
        steady = {"warm_steps": n_warm, "warm_s": warm_s, "per_kernel": pk2,
                  "ms_step": wall2 * 1e3 / steps}
    # outputs of the timed run must be finite (parity itself is the tests' job)
    check = {"o_finite": bool(torch.isfinite(o.float()).all()),
             "lse_finite_or_neg_inf": bool((torch.isfinite(lse) | (lse == -float("inf"))).all())}
    if w.backward:
        check["grads_finite"] = bool(all(torch.isfinite(t.float()).all()
                                         for t in (dq, dk, dv)))
    pairs = visible_pairs(w, inp["kv_len"], inp.get("block_mask"))
    return {"inp": inp, "names": names, "per_kernel": per_kernel,
            "ms_step": wall * 1e3 / steps, "pairs": pairs, "fp8": fp8,
            "dropout": dr, "check": check, "steps": steps, "warmup": warmup,
            "steady": steady}


def record_calls(fa, stage):
    """The C calls (function, argument tuple) that one binding call makes,
    recorded instead of executed."""
    real = fa.lib()
    rec = []

    class Recorder:
        def __getattr__(self, name):
            fn = getattr(real, name)

            def call(*args):
                rec.append((fn, args))
                return 0
            return call
    saved = fa._lib
    fa._lib = Recorder()
    try:
        stage()
    finally:
        fa._lib = saved
    return rec


def _peak(w: S.Workload, fp8: bool) -> float:
    return (PEAK_F32_TFLOPS if w.dtype == "f32" else
            PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS)


def result_line(w: S.Workload, res: dict, args) -> dict:
    """The JSON line of one timed workload (without per_config)."""
    import torch
    dev = torch.device("cuda:0")
    per_kernel, ms_step, pairs = res["per_kernel"], res["ms_step"], res["pairs"]
    names, fp8, dr, inp = res["names"], res["fp8"], res["dropout"], res["inp"]
    fwd_flops = linear_flops(w) if w.linear else 4.0 * w.d * pairs
    bwd_flops = ((linear_bwd_flops(w) if w.linear else 10.0 * w.d * pairs)
                 if w.backward else 0.0)
    step_flops = fwd_flops + bwd_flops
    value = step_flops / (ms_step * 1e-3) / 1e12
    peak = _peak(w, fp8)

    if w.backward and w.linear:
        # fa_linear_bwd: three chunkwise passes (dQ; dK and dV reversed)
        dom, dom_flops, src = ("linear_bwd", bwd_flops,
                               ["fa_linear.hip", "fa_common.h"])
    elif w.backward:
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
    if traffic is not None:
        roofline["traffic_gb_per_s"] = round(traffic / (dom_ms * 1e-3) / 1e9, 1)

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
        "n_gpus": 1, "steps": res["steps"], "warmup": res["warmup"],
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
        "fwd_tflops": round(fwd_flops / (per_kernel["fwd_fp8" if fp8 else
                                                    "linear_fwd" if w.linear
                                                    else "fwd"]
                                         * 1e-3) / 1e12, 2),
        "roofline": roofline,
        "mfma_ceiling": ceiling,
        "cpu_baseline": cpu,
        "sanity": res["check"],
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
    st = res.get("steady")
    if st:
        spk, sms = st["per_kernel"], st["ms_step"]
        sd = spk[dom]
        sa = (algorithmic_bytes(w, dom) / (sd * 1e-3) / 1e9
              if roofline["unit"] == "GB/s" else dom_flops / (sd * 1e-3) / 1e12)
        sv = step_flops / (sms * 1e-3) / 1e12
        out["steady_state"] = {
            "what": ("the same steps timed again after more untimed steps, "
                     "at the clock the GPU sustains under load; value and "
                     "roofline above are the measurement after --warmup steps"),
            "warm_steps": st["warm_steps"], "warm_s": round(st["warm_s"], 2),
            "value": round(sv, 2), "frac_of_peak": round(sv / peak, 4),
            "ms_per_step": round(sms, 4),
            "kernel_ms": {n: round(t, 4) for n, t in spk.items()},
            "dominant": {"kernel": dom, "achieved": round(sa, 2),
                         "unit": roofline["unit"],
                         "frac": round(sa / roofline["peak"], 4)}}
    return out


def oracle_timing(w: S.Workload, inp: dict, runs: int, max_heads=None):
    """Seconds of the fp64 oracle on the workload (its first max_heads
    (b, h) heads of batch entry 0 when given, else all of it), median of
    `runs` runs; returns (seconds, heads timed, algorithmic FLOP timed)."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    kv = inp["kv_len"]
    q, k, v = inp["q"], inp["k"], inp["v"]
    do = inp.get("do")
    B = w.B
    if max_heads is not None:
        q, k, v = (a[:1, :max_heads] for a in (q, k, v))
        do = None if do is None else do[:1, :max_heads]
        kv = None if kv is None else kv[:1]
        B = 1
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        oracle.attention_fwd(q, k, v, inp["scale"], inp["causal"], kv,
                             workers=cores)
        if w.backward:
            oracle.attention_bwd(q, k, v, do, inp["scale"], inp["causal"], kv,
                                 workers=cores)
        ts.append(time.perf_counter() - t0)
    nh = q.shape[0] * q.shape[1]
    sw = S.Workload(w.name, B, q.shape[1], w.N, w.d, w.dtype, w.causal,
                    w.seeds, w.backward)
    flops = visible_pairs(sw, kv) * w.d * (4 + (10 if w.backward else 0))
    return float(np.median(ts)), nh, flops


def per_config(dev, args, head_res: dict, head_out: dict) -> dict:
    """Every synthetic config the metric is quoted on: algorithmic TFLOP/s,
    fraction of its peak, kernel time, and the fp64 oracle timed on the
    host cores of this run (configs 1-3 whole, median of 3 runs; configs 4
    and 5 on a bounded sample of heads, one run); with --steady-s, each
    config's rate under sustained load as well.  The configs other than the
    headline's take their wall clock over steps without per-kernel events
    (time_workload's bare_wall)."""
    cores = len(os.sched_getaffinity(0))
    table = {}
    for num, name in CONFIGS:
        w = S.WORKLOADS[name]
        if name == head_out["config"]["workload"]:
            res, line = head_res, head_out
        else:
            res = time_workload(w, dev, args.steps, args.warmup,
                                steady_s=args.steady_s, bare_wall=True)
            fwd_flops = 4.0 * w.d * res["pairs"]
            line = {"value": fwd_flops / (res["ms_step"] * 1e-3) / 1e12,
                    "ms_per_step": res["ms_step"]}
        fwd_ms = res["per_kernel"]["fwd"]
        fwd_flops = 4.0 * w.d * res["pairs"]
        peak = _peak(w, False)
        ent = {"workload": name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
               "dtype": w.dtype, "causal": w.causal,
               "pass": "forward+backward" if w.backward else "forward",
               "visible_pairs": res["pairs"],
               "tflops": round(line["value"], 2),
               "frac_of_peak": round(line["value"] / peak, 4),
               "peak_tflops": peak, "ms_per_step": round(line["ms_per_step"], 4),
               "kernel_ms": {n: round(t, 4) for n, t in res["per_kernel"].items()},
               "fwd_tflops": round(fwd_flops / (fwd_ms * 1e-3) / 1e12, 2),
               "fwd_frac_of_peak": round(fwd_flops / (fwd_ms * 1e-3) / 1e12 / peak, 4),
               "wall": ("steps with per-kernel events" if res is head_res else
                        "steps without events; kernel_ms from as many more "
                        "steps with events")}
        if w.backward:
            bwd_ms = sum(res["per_kernel"][n] for n in res["names"][1:])
            bt = 10.0 * w.d * res["pairs"] / (bwd_ms * 1e-3) / 1e12
            ent["bwd_tflops"] = round(bt, 2)
            ent["bwd_frac_of_peak"] = round(bt / peak, 4)
        st = res.get("steady")
        if st:
            step_flops = (14.0 if w.backward else 4.0) * w.d * res["pairs"]
            sv = step_flops / (st["ms_step"] * 1e-3) / 1e12
            sf = fwd_flops / (st["per_kernel"]["fwd"] * 1e-3) / 1e12
            ent["steady_state"] = {
                "warm_steps": st["warm_steps"], "tflops": round(sv, 2),
                "frac_of_peak": round(sv / peak, 4),
                "fwd_tflops": round(sf, 2), "fwd_frac_of_peak": round(sf / peak, 4),
                "kernel_ms": {n: round(t, 4) for n, t in st["per_kernel"].items()}}
        if not args.no_cpu_baseline:
            if num <= 3:
                log(f"[bench] oracle on config {num} (3 runs)")
                sec, nh, fl = oracle_timing(w, res["inp"], 3)
                sample = f"whole workload ({nh} heads), median of 3 runs"
            elif num == 4:
                log(f"[bench] oracle on config {num} (1 head)")
                sec, nh, fl = oracle_timing(w, res["inp"], 1, max_heads=1)
                sample = "1 of 12 heads (all 23400 rows), one run"
            else:
                cb = head_out.get("cpu_baseline") or {}
                sec, nh, fl = None, None, None
                sample = cb.get("sample", "")
                ent["oracle"] = {"tflops": cb.get("value"), "sample": sample,
                                 "cores": cores}
            if sec is not None:
                ent["oracle"] = {"seconds": round(sec, 3), "heads": nh,
                                 "tflops": fl / sec / 1e12, "cores": cores,
                                 "sample": sample}
            if ent["oracle"].get("tflops"):
                ent["gpu_over_oracle"] = round(
                    ent["tflops"] / ent["oracle"]["tflops"], 1)
        table[str(num)] = ent
        del res
    return table


if __name__ == "__main__":
    sys.exit(main())
