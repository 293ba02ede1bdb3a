"""CPU model of the FP8 forward with incoherent processing (fp64 attention on
the quantised operands) -- TEST INFRASTRUCTURE ONLY.

Like the rest of this package it is imported only by the tests, the smoke
check and the benchmark's CPU-baseline leg; it shares no code with the HIP
library or its binding.

Page cited: [MM] "Is a full-day context better than a 10-minute context?
Flash attention and the sequence-length question" (marketmaker.cc blog),
section "FA3: Hopper", item 3.  The page says that FP8 attention is hurt by
outliers, and that FA3 rotates the vectors at random before quantising them
block by block, which spreads an outlier's magnitude over all coordinates
and gives a smaller numerical error than plain FP8.  It gives no formulas.
The readings taken here (each also listed in the design notes):

  * The random orthogonal map is a randomised Hadamard transform applied to
    every row of Q and of K: multiply coordinate c by a random sign s_c,
    then apply the Sylvester-Hadamard matrix H_d (entries +-1) by the fast
    Walsh-Hadamard transform.  R = diag(s) H_d satisfies R R^T = d I, so
    (Q R)(K R)^T = d Q K^T and the scores are taken with scale / d.  The
    signs are an input (the random draw is passed in).  V is not rotated.
  * The transform runs in float32, stage by stage: stage t = 0, 1, ...
    pairs coordinates i and i + 2^t (bit t of i clear) into (a + b, a - b).
    The order is part of the definition because the quantisation codes
    below are decided on its float32 results.
  * Block-wise quantisation: each block of 32 consecutive values -- along
    the head dimension for the rows of Q and K, along the keys for each
    channel of V -- shares one power-of-two scale 2^e, with e the smallest
    integer such that the block's largest magnitude is at most 448 * 2^e
    (448 is the largest finite FP8 E4M3 value), clamped to [-127, 127]
    (-127 for an all-zero block).  Each value x becomes the E4M3 code of
    x * 2^-e, rounded to nearest with ties to even (the product is exact:
    only the exponent changes).  Keys past N count as zeros.
  * Attention is then the plain definition (oracle.attention) in fp64 on the
    dequantised operands.  The GPU also rounds the softmax weights to E4M3
    before the P V product; that rounding depends on the kernel's running
    reference and is not modelled here (the tests bound it): parity
    unpinned for that step.
"""
from __future__ import annotations

import numpy as np

from oracle.attention import attention_fwd

__all__ = ["E4M3_MAX", "MX_BLOCK", "e4m3_decode", "e4m3_encode",
           "fwht_f32", "rotate_f32", "mx_exponent", "mx_quantize",
           "mx_dequantize", "fp8_forward"]

E4M3_MAX = 448.0
MX_BLOCK = 32


def _decode_table() -> np.ndarray:
    """Value of every E4M3 (OCP "fn" variant) byte: 1 sign bit, 4 exponent
    bits with bias 7, 3 mantissa bits; exponent 0 is subnormal
    (mantissa/8 * 2^-6); byte 0x7F / 0xFF is NaN and there is no infinity."""
    t = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            t[c] = np.nan
        elif e == 0:
            t[c] = sign * (m / 8.0) * 2.0 ** -6
        else:
            t[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


_TABLE = _decode_table()
# Non-negative finite values (codes 0x00..0x7E), increasing with the code.
_POS = _TABLE[:0x7F]


def e4m3_decode(codes) -> np.ndarray:
    """float64 values of E4M3 bytes."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    """E4M3 byte of each float32 value, round to nearest, ties to even.

    |x| must not exceed 448 (the block scale guarantees it).  The sign is
    kept, so a negative value that rounds to zero gives 0x80.
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    if np.any(~np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_encode: value outside [-448, 448]")
    a = np.abs(x)
    # Spacing of E4M3 values around a: 2^-9 below 2^-6 (subnormals), else
    # 2^(floor(log2 a) - 3).
    _, ex = np.frexp(np.where(a > 0, a, 1.0))          # a = f 2^ex, f in [.5, 1)
    step = np.where(a < 2.0 ** -6, 2.0 ** -9, np.ldexp(1.0, ex - 1 - 3))
    n = np.rint(a / step)                              # ties to even (exact a/step)
    val = n * step
    code = np.searchsorted(_POS, val)
    assert np.all(_POS[code] == val)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def fwht_f32(x) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform of the last axis in float32,
    stage t = 0, 1, ... pairing i and i + 2^t into (a + b, a - b)."""
    y = np.array(x, dtype=np.float32, copy=True)
    d = y.shape[-1]
    assert d & (d - 1) == 0
    h = 1
    while h < d:
        z = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a = z[..., 0, :]
        b = z[..., 1, :]
        y = np.stack([a + b, a - b], axis=-2).reshape(y.shape)
        h *= 2
    return y


def rotate_f32(x, signs) -> np.ndarray:
    """x R with R = diag(signs) H_d, in float32 (sign flips are exact)."""
    s = np.where(np.asarray(signs) < 0, -1.0, 1.0).astype(np.float32)
    return fwht_f32(np.asarray(x, dtype=np.float32) * s)


def mx_exponent(amax) -> np.ndarray:
    """Smallest integer e with amax <= 448 * 2^e, clamped to [-127, 127];
    -127 where amax = 0."""
    a = np.asarray(amax, dtype=np.float64)
    f, ex = np.frexp(np.where(a > 0, a, 1.0))          # a = (2f) 2^(ex-1)
    # 448 = 1.75 * 2^8: a fits 2^(ex-1-8) * 448 iff its mantissa 2f <= 1.75.
    e = np.where(2.0 * f <= 1.75, ex - 1 - 8, ex - 1 - 7)
    e = np.where(a > 0, e, -127)
    return np.clip(e, -127, 127).astype(np.int64)


def mx_quantize(x):
    """Quantise the last axis (a multiple of 32 long) in blocks of 32.

    Returns (codes uint8 of x's shape, e int64 [..., n / 32])."""
    x = np.asarray(x, dtype=np.float32)
    n = x.shape[-1]
    assert n % MX_BLOCK == 0
    blocks = x.reshape(x.shape[:-1] + (n // MX_BLOCK, MX_BLOCK))
    e = mx_exponent(np.abs(blocks.astype(np.float64)).max(axis=-1))
    scaled = np.ldexp(blocks.astype(np.float64), -e[..., None])
    assert np.all(scaled.astype(np.float32) == scaled)  # exponent shift only
    codes = e4m3_encode(scaled.astype(np.float32))
    return codes.reshape(x.shape), e


def mx_dequantize(codes, e) -> np.ndarray:
    """float64 values of quantised blocks (inverse of mx_quantize's map)."""
    codes = np.asarray(codes, dtype=np.uint8)
    n = codes.shape[-1]
    v = e4m3_decode(codes).reshape(codes.shape[:-1] + (n // MX_BLOCK, MX_BLOCK))
    return np.ldexp(v, np.asarray(e)[..., None]).reshape(codes.shape)


def fp8_forward(q, k, v, scale, causal=False, signs=None, workers=None):
    """FP8 forward of the model above.

    q, k, v: [B, H, N, d] holding exactly the (bf16) values the GPU sees;
    signs: None (no rotation: plain FP8) or d values whose sign is used.
    Returns a dict: o, lse (fp64, [B,H,N,d] / [B,H,N]) and the quantised
    operands q_codes, k_codes [B,H,N,d] with q_exp, k_exp [B,H,N,d/32],
    v_codes [B,H,d,Np] with v_exp [B,H,d,Np/32] (Np = N rounded up to 32).
    """
    q = np.asarray(q, dtype=np.float32)
    k = np.asarray(k, dtype=np.float32)
    v = np.asarray(v, dtype=np.float32)
    B, H, N, d = q.shape
    sc = float(np.float32(scale))
    if signs is not None:
        q = rotate_f32(q, signs)
        k = rotate_f32(k, signs)
        sc = sc / d
    qc, qe = mx_quantize(q)
    kc, ke = mx_quantize(k)
    Np = -(-N // MX_BLOCK) * MX_BLOCK
    vt = np.zeros((B, H, d, Np), dtype=np.float32)
    vt[..., :N] = np.swapaxes(v, -1, -2)
    vc, ve = mx_quantize(vt)
    qh = mx_dequantize(qc, qe)
    kh = mx_dequantize(kc, ke)
    vh = np.swapaxes(mx_dequantize(vc, ve), -1, -2)[:, :, :N]
    o, lse = attention_fwd(qh, kh, vh, sc, causal, workers=workers)
    return {"o": o, "lse": lse, "q_codes": qc, "q_exp": qe, "k_codes": kc,
            "k_exp": ke, "v_codes": vc, "v_exp": ve, "scale_used": sc,
            "q_deq": qh, "k_deq": kh, "v_deq": vh}
