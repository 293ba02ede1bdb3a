"""Seeded synthetic inputs for the attention workloads.

This module holds no attention arithmetic.  It draws iid standard-normal
tensors from numpy's PCG64 generator, rounds them to bfloat16 (round to
nearest, ties to even, on the float32 bit pattern), adds the slow sinusoidal
key drift of the long-context workload, and draws key-padding lengths.  The
fp64 oracle's tests and the HIP path's tests and benchmark both take their
inputs from here, so both sides see identical bits.

Shapes follow the public workloads that the FlashAttention pages measure on
("Paper summary: FlashAttention", zenn.dev, section Overview: BERT-large at
sequence length 512, GPT-2 at 1K, Long Range Arena at 1K-4K) and the trading
day of "Is a full-day context better than a 10-minute context? Flash attention
and the sequence-length question" (marketmaker.cc, introduction: 23,400
one-second steps, 12 heads).  No dataset is read: every tensor is synthetic.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "bf16_round_bits", "bf16_bits_to_f32", "normal",
    "make_inputs", "make_case", "block_mask", "rotation_signs",
    "outlier_channels",
]


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bfloat16 bit patterns, round-to-nearest-even.

    Inputs here are finite normals, so NaN handling is not needed; an Inf
    input stays Inf (0x7f800000 has zero low bits).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def normal(seed: int, shape) -> np.ndarray:
    """iid N(0,1) float32 from numpy's default generator (PCG64) at `seed`."""
    return np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "f32" or "bf16"
    causal: bool
    seeds: tuple          # (q, k, v) or (q, k, v, dO)
    backward: bool = False
    kv_len_seed: int | None = None   # key-padding lengths drawn from this seed
    kv_len_range: tuple = (0, 0)     # inclusive [lo, hi]
    drift_period: float = 0.0        # sinusoidal drift on K (0 = none)
    drift_amp: float = 0.0
    block_seed: int | None = None    # block-sparse mask drawn from this seed
    block_density: float = 0.0
    sign_seed: int | None = None     # FP8 path: rotation signs from this seed
    linear: bool = False             # causal linear attention (no softmax)
    drop_p: float = 0.0              # attention dropout probability
    drop_seed: int | None = None     # 64-bit generator key of the dropout mask
    description: str = ""

    @property
    def scale(self) -> float:
        """1/sqrt(d) rounded to float32 (the value the C ABI receives)."""
        return float(np.float32(1.0 / math.sqrt(self.d)))


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_f32", 1, 1, 256, 64, "f32", False, (101, 102, 103),
                 description="tiny fp32 non-causal forward"),
        Workload("gpt2_causal", 8, 12, 1024, 64, "bf16", True, (201, 202, 203),
                 description="GPT-2-small-shaped causal forward"),
        Workload("gpt2_causal_fwd_bwd", 8, 12, 1024, 64, "bf16", True,
                 (201, 202, 203, 204), backward=True,
                 description="GPT-2-small-shaped causal forward + backward "
                             "(a training step's attention)"),
        Workload("bert_keypad", 16, 16, 512, 64, "bf16", False, (301, 302, 303),
                 kv_len_seed=309, kv_len_range=(256, 512),
                 description="BERT-large-shaped forward with key padding"),
        Workload("tradingday_causal", 1, 12, 23400, 64, "bf16", True,
                 (401, 402, 403), drift_period=390.0, drift_amp=0.5,
                 description="one trading day at 1-s steps, causal forward"),
        Workload("causal_fwd_bwd_d128", 4, 16, 4096, 128, "bf16", True,
                 (501, 502, 503, 504), backward=True,
                 description="causal forward + backward, head dim 128"),
        Workload("blocksparse_d128", 4, 16, 4096, 128, "bf16", False,
                 (601, 602, 603), block_seed=609, block_density=0.5,
                 description="block-sparse forward, half of the 256x128 "
                             "blocks kept per head, head dim 128"),
        Workload("blocksparse_fwd_bwd_d128", 4, 16, 4096, 128, "bf16", False,
                 (601, 602, 603, 604), backward=True, block_seed=609,
                 block_density=0.5,
                 description="block-sparse forward + backward, the blocks "
                             "of blocksparse_d128"),
        Workload("fp8_causal_d128", 4, 16, 4096, 128, "bf16", True,
                 (701, 702, 703), sign_seed=709,
                 description="FP8 causal forward with incoherent processing "
                             "(bf16 inputs quantised on the GPU), head dim "
                             "128"),
        Workload("linear_causal_d128", 4, 16, 4096, 128, "bf16", True,
                 (801, 802, 803), linear=True,
                 description="causal linear attention (chunkwise), head dim "
                             "128"),
        Workload("linear_causal_fwd_bwd_d128", 4, 16, 4096, 128, "bf16", True,
                 (801, 802, 803, 804), backward=True, linear=True,
                 description="causal linear attention forward + backward "
                             "(chunkwise), head dim 128"),
        Workload("dropout_causal_fwd_bwd_d128", 4, 16, 4096, 128, "bf16", True,
                 (901, 902, 903, 904), backward=True, drop_p=0.1,
                 drop_seed=0x243F6A8885A308D3,
                 description="causal forward + backward with attention "
                             "dropout p = 0.1, head dim 128"),
    ]
}


def _finish(arr32: np.ndarray, dtype: str):
    """Return (values as float32 exactly representable in dtype, raw bits)."""
    if dtype == "bf16":
        bits = bf16_round_bits(arr32)
        return bf16_bits_to_f32(bits), bits
    if dtype == "f32":
        a = np.ascontiguousarray(arr32, dtype=np.float32)
        return a, a
    raise ValueError(dtype)


def make_inputs(w: Workload | str, heads: slice | None = None) -> dict:
    """Generate the inputs of workload `w`.

    Returns a dict with keys q, k, v (and do when w.backward): float32 arrays
    of shape [B,H,N,d] holding exactly the values the GPU sees; q_bits, ...
    with the raw bits to upload (uint16 for bf16, float32 for f32); kv_len
    (int32 [B] or None); scale; causal; dtype.

    `heads` optionally keeps a slice of the H axis (after generation, so the
    kept values are identical to the full workload's).
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    shape = (w.B, w.H, w.N, w.d)
    out = {"scale": w.scale, "causal": w.causal, "dtype": w.dtype,
           "workload": w.name}
    names = ["q", "k", "v", "do"][: len(w.seeds)]
    for name, seed in zip(names, w.seeds):
        a = normal(seed, shape)
        if name == "k" and w.drift_amp:
            t = np.arange(w.N, dtype=np.float64)
            drift = (w.drift_amp * np.sin(2.0 * np.pi * t / w.drift_period)
                     ).astype(np.float32)
            a += drift[None, None, :, None]
        if heads is not None:
            a = np.ascontiguousarray(a[:, heads])
        vals, bits = _finish(a, w.dtype)
        out[name] = vals
        out[name + "_bits"] = bits
    if w.block_seed is not None:
        out["block_mask"] = block_mask(w.block_seed, w.H, w.N, w.block_density)
        if heads is not None:
            out["block_mask"] = np.ascontiguousarray(out["block_mask"][heads])
    if w.sign_seed is not None:
        out["signs"] = rotation_signs(w.sign_seed, w.d)
    if w.drop_seed is not None:
        out["dropout"] = {"p": w.drop_p, "seed": w.drop_seed, "offset": 0}
    if w.kv_len_seed is not None:
        lo, hi = w.kv_len_range
        out["kv_len"] = np.random.default_rng(w.kv_len_seed).integers(
            lo, hi + 1, w.B).astype(np.int32)
    else:
        out["kv_len"] = None
    return out


def block_mask(seed: int, H: int, N: int, density: float,
               bq: int = 256, bk: int = 128) -> np.ndarray:
    """Seeded block mask, uint8 [H, ceil(N/bq), ceil(N/bk)]: each block is
    kept with probability `density`, and the block holding the diagonal of
    each block row is always kept (so every query row sees some key)."""
    tq, tk = -(-N // bq), -(-N // bk)
    m = (np.random.default_rng(seed).random((H, tq, tk)) < density)
    r = np.arange(tq)
    m[:, r, np.minimum(r * bq // bk, tk - 1)] = True
    return m.astype(np.uint8)


def rotation_signs(seed: int, d: int) -> np.ndarray:
    """Seeded random signs (int8, +1 or -1) for the FP8 path's rotation."""
    return np.where(np.random.default_rng(seed).random(d) < 0.5, -1,
                    1).astype(np.int8)


def outlier_channels(seed: int, d: int, n: int) -> np.ndarray:
    """Seeded choice of n distinct feature channels (sorted int array)."""
    return np.sort(np.random.default_rng(seed).choice(d, n, replace=False))


def make_case(B, H, N, d, dtype="bf16", causal=False, seed=0, kv_len=None,
              backward=False, q_scale=1.0, scale=None, outliers=0,
              outlier_scale=1.0) -> dict:
    """Small seeded case for parity tests; same dict layout as make_inputs.

    `q_scale` multiplies Q before rounding (large-magnitude score tests).
    `kv_len` may be None, an int (same for every batch), or a sequence.
    `outliers` > 0 multiplies that many feature channels (the same ones in
    Q and K, chosen by `outlier_channels(seed, d, outliers)`) by
    `outlier_scale` before rounding: outlier features shared by queries and
    keys.
    """
    shape = (B, H, N, d)
    out = {"causal": causal, "dtype": dtype, "workload": "case"}
    out["scale"] = float(np.float32(1.0 / math.sqrt(d))) if scale is None \
        else float(np.float32(scale))
    names = ["q", "k", "v", "do"] if backward else ["q", "k", "v"]
    for i, name in enumerate(names):
        a = normal(seed * 16 + i, shape)
        if name == "q" and q_scale != 1.0:
            a = (a * np.float32(q_scale)).astype(np.float32)
        if outliers and name in ("q", "k"):
            ch = outlier_channels(seed, d, outliers)
            a[..., ch] *= np.float32(outlier_scale)
        vals, bits = _finish(a, dtype)
        out[name] = vals
        out[name + "_bits"] = bits
    if kv_len is None:
        out["kv_len"] = None
    elif np.isscalar(kv_len):
        out["kv_len"] = np.full(B, int(kv_len), dtype=np.int32)
    else:
        out["kv_len"] = np.asarray(kv_len, dtype=np.int32)
    return out
