"""fp64 CPU oracle for attention with dropout on the weights -- TEST
INFRASTRUCTURE ONLY.

Like the rest of this package it is imported only by the tests, the smoke
check and the benchmark's CPU-baseline leg; it shares no code with the HIP
library or its binding.

Pages cited:
  [MM] "Is a full-day context better than a 10-minute context? Flash
       attention and the sequence-length question" (marketmaker.cc blog),
       "Integration": the framework call takes a dropout probability
       alongside q, k, v and the causal flag.  The pages say nothing more
       about it.

Readings (also in the design notes):
  * Dropout acts on the normalised attention weights, as the framework call
    does: O = (P o Z / keep) V with P = softmax(scale Q K^T) (masked as in
    oracle.attention), Z a 0/1 keep mask and keep the keep probability.
    LSE is the log-sum-exp of the undropped scores (what the backward needs
    to recompute P).
  * The random numbers come from Philox4x32-10, the counter-based generator
    of Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as
    1, 2, 3" (SC 2011): a 128-bit counter and a 64-bit key give four 32-bit
    words after ten rounds of the Philox S-box (two 32x32->64-bit products
    with the constants below, xor with the other words and the round key)
    and a Weyl-sequence key schedule.
  * Element (b, h, i, j) reads one byte: the counter is
    (j // 4, i // 4, b*H + h, offset) and the key (seed mod 2^32,
    seed // 2^32); the byte is byte (j mod 4) (least significant first) of
    word (i mod 4) of the output.  One generator call thus serves a 4 x 4
    block of (query, key) pairs.
  * The drop probability is applied in steps of 1/256: p8 = round(256 p),
    0 <= p8 <= 255; an element is kept iff its byte >= p8, so the keep
    probability is (256 - p8) / 256 and kept weights are divided by it.
  * Backward: the analytic gradient of <dO, O> for a fixed mask Z:
        dV = (P o Z / keep)^T dO,  dP = (dO V^T) o Z / keep,
        D_i = sum_j P_ij dP_ij (= dO_i . O_i),  dS = P o (dP - D),
        dQ = scale dS K,  dK = scale dS^T Q.
"""
from __future__ import annotations

import numpy as np

__all__ = ["philox4x32_10", "threshold", "keep_prob", "keep_mask",
           "attention_dropout_fwd", "attention_dropout_bwd"]

# Philox4x32 constants (the paper's multipliers and Weyl key increments).
_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = 0x9E3779B9
_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32 with ten rounds on arrays of counters (any broadcastable
    shapes); key words k0, k1 are Python ints.  Returns four uint32 arrays.

    Round: with the current counter (x0, x1, x2, x3) and round key
    (r0, r1), form the 64-bit products M0 x0 and M1 x2; the new counter is
    (hi(M1 x2) ^ x1 ^ r0, lo(M1 x2), hi(M0 x0) ^ x3 ^ r1, lo(M0 x0)).  The
    round key starts at (k0, k1) and grows by (W0, W1) mod 2^32 after every
    round."""
    x = [np.asarray(c, dtype=np.uint64) & _MASK32 for c in (c0, c1, c2, c3)]
    x = np.broadcast_arrays(*x)
    x = [a.copy() for a in x]
    r0, r1 = int(k0) & 0xFFFFFFFF, int(k1) & 0xFFFFFFFF
    for _ in range(10):
        p0 = _M0 * x[0]                      # < 2^64: exact in uint64
        p1 = _M1 * x[2]
        x = [(p1 >> np.uint64(32)) ^ x[1] ^ np.uint64(r0),
             p1 & _MASK32,
             (p0 >> np.uint64(32)) ^ x[3] ^ np.uint64(r1),
             p0 & _MASK32]
        r0 = (r0 + _W0) & 0xFFFFFFFF
        r1 = (r1 + _W1) & 0xFFFFFFFF
    return [a.astype(np.uint32) for a in x]


def threshold(p: float) -> int:
    """Byte threshold p8 = round(256 p) of the probability given as a
    float32 (ties to even, as numpy rounds)."""
    p8 = int(np.rint(256.0 * float(np.float32(p))))
    if not (0 <= p8 <= 255):
        raise ValueError("drop probability must round to 0..255 / 256")
    return p8


def keep_prob(p8: int) -> float:
    return (256 - int(p8)) / 256.0


def keep_mask(seed: int, offset: int, p8: int, bh: int, rows, n_keys: int):
    """Boolean [len(rows), n_keys]: the keep mask Z of head bh (= b*H + h)
    for the given query rows.  One generator call per (row's query group,
    key group); row i takes word i % 4 of its calls, key j byte j % 4."""
    rows = np.asarray(rows, dtype=np.int64)
    n_kb = -(-int(n_keys) // 4)
    kb = np.arange(n_kb, dtype=np.int64)[None, :]
    qb = (rows // 4)[:, None]
    words = philox4x32_10(kb, qb, np.uint64(bh), np.uint64(offset),
                          int(seed) & 0xFFFFFFFF, (int(seed) >> 32) & 0xFFFFFFFF)
    w = np.stack(words, axis=0)                         # [4, rows, key groups]
    word = w[(rows % 4)[:, None], np.arange(len(rows))[:, None], kb]  # [rows, groups]
    shifts = np.arange(4, dtype=np.uint32) * np.uint32(8)
    byte = (word[:, :, None] >> shifts) & np.uint32(0xFF)   # [rows, groups, 4]
    return (byte >= np.uint32(p8)).reshape(len(rows), 4 * n_kb)[:, :n_keys]


def _probs(qh, kh, scale, causal, rows):
    """Two-pass softmax rows of one head: (P, m) with P [rows, N]."""
    s = scale * (qh[rows] @ kh.T)
    if causal:
        s = np.where(np.arange(kh.shape[0])[None, :] <= rows[:, None], s, -np.inf)
    m = s.max(axis=1)
    e = np.exp(s - np.where(np.isfinite(m), m, 0.0)[:, None])
    l = e.sum(axis=1)
    return e / np.where(l > 0, l, 1.0)[:, None], m, l


def attention_dropout_fwd(q, k, v, scale, causal, p8, seed, offset=0,
                          rows=None, bh0=0):
    """O, LSE of softmax attention with dropout on the weights (float64).

    q, k, v: [B, H, N, d]; rows: optional query indices (then only those
    rows are computed).  The mask of head (b, h) is that of generator head
    index bh0 + b*H + h (bh0 places a slice of heads within a larger
    batch)."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, N, d = q.shape
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    kp = keep_prob(p8)
    o = np.zeros((B, H, len(rows), v.shape[-1]))
    lse = np.zeros((B, H, len(rows)))
    for b in range(B):
        for h in range(H):
            p, m, l = _probs(q[b, h], k[b, h], float(scale), causal, rows)
            z = keep_mask(seed, offset, p8, bh0 + b * H + h, rows, N)
            o[b, h] = (p * z / kp) @ v[b, h]
            lse[b, h] = m + np.log(l)
    return o, lse


def attention_dropout_bwd(q, k, v, do, scale, causal, p8, seed, offset=0,
                          bh0=0):
    """Analytic (dQ, dK, dV) of <dO, O> for attention with dropout, fixed Z
    (heads numbered as in attention_dropout_fwd)."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    B, H, N, d = q.shape
    scale = float(scale)
    kp = keep_prob(p8)
    rows = np.arange(N)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            p, _, _ = _probs(q[b, h], k[b, h], scale, causal, rows)
            z = keep_mask(seed, offset, p8, bh0 + b * H + h, rows, N)
            dv[b, h] = (p * z / kp).T @ do[b, h]
            dp = (do[b, h] @ v[b, h].T) * z / kp
            D = (p * dp).sum(axis=1)
            ds = p * (dp - D[:, None])
            dq[b, h] = scale * (ds @ k[b, h])
            dk[b, h] = scale * (ds.T @ q[b, h])
    return dq, dk, dv
