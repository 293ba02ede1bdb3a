"""fp64 CPU oracle for causal linear attention -- TEST INFRASTRUCTURE ONLY.

Like the rest of this package it is imported only by the tests, the smoke
check and the benchmark's CPU-baseline leg; it shares no code with the HIP
library or its binding.

Pages cited:
  [LA2] "Lightning Attention-2: A Free Lunch for Handling Unlimited Sequence
        Lengths in Large Language Models" (abstract page): linear attention
        processed in blocks, with ordinary attention-style computation inside
        a block and the linear-attention kernel trick between blocks.
  [GLA] "[Paper review] Gated Linear Attention Transformers with
        Hardware-Efficient Training" (review page), abstract and "proposed
        method": linear attention is also an RNN with a matrix-valued hidden
        state; FLASHLINEARATTENTION combines a recurrence between chunks with
        parallel computation inside a chunk.

What it computes.  The pages give no formulas.  The reading taken (also in
the design notes): causal linear attention without softmax, normalisation,
decay or gates,
    O_i = scale * sum_{j <= i} (q_i . k_j) v_j,   i.e.  O = scale * tril(Q K^T) V,
per (batch, head), the form that both the block split of [LA2] and the
chunkwise/recurrent forms of [GLA] compute exactly.  The oracle is that
quadratic definition in float64, rows in chunks (each row computed whole).

Backward.  [LA2]'s abstract says the tiling serves the backward pass as
well as the forward, and [GLA] presents the chunkwise form as the route to
hardware-efficient training; neither gives the gradient.  The oracle is the
analytic gradient of <dO, O> for O = scale * A V with A = tril(Q K^T):
    dV = scale * A^T dO,   dA = scale * tril(dO V^T),
    dQ = dA K,             dK = dA^T Q,
i.e. dQ_i = scale sum_{j<=i} (dO_i . v_j) k_j,
     dK_j = scale sum_{i>=j} (dO_i . v_j) q_i,
     dV_j = scale sum_{i>=j} (q_i . k_j) dO_i,
evaluated in float64 over row chunks (dK and dV accumulate over them).
"""
from __future__ import annotations

import numpy as np

__all__ = ["linear_attention_fwd", "linear_attention_bwd", "linear_pairs"]


def linear_attention_fwd(q, k, v, scale, row_chunk=1024, rows=None):
    """O = scale * tril(Q K^T) V for q, k, v [B, H, N, d]; float64 out.

    rows: optional 1-D array of query indices; then only those rows are
    computed and the output has that many rows."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    scale = float(scale)
    B, H, N, d = q.shape
    idx = np.arange(N) if rows is None else np.asarray(rows)
    o = np.zeros((B, H, len(idx), v.shape[-1]), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, len(idx), row_chunk):
                r1 = min(len(idx), r0 + row_chunk)
                rr = idx[r0:r1]
                n1 = int(rr.max()) + 1
                a = q[b, h, rr] @ k[b, h, :n1].T             # [rows, keys]
                i = rr[:, None]
                j = np.arange(n1)[None, :]
                a = np.where(j <= i, a, 0.0)
                o[b, h, r0:r1] = scale * (a @ v[b, h, :n1])
    return o


def linear_attention_bwd(q, k, v, do, scale, row_chunk=1024):
    """Gradients (dQ, dK, dV) of <dO, O> for O = scale * tril(Q K^T) V;
    q, k, v, do [B, H, N, d]; float64 out, [B, H, N, d] each."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    scale = float(scale)
    B, H, N, d = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, row_chunk):
                r1 = min(N, r0 + row_chunk)
                i = np.arange(r0, r1)[:, None]
                j = np.arange(r1)[None, :]
                vis = j <= i                                  # rows r0..r1-1
                a = np.where(vis, q[b, h, r0:r1] @ k[b, h, :r1].T, 0.0)
                da = np.where(vis, scale * (do[b, h, r0:r1] @ v[b, h, :r1].T), 0.0)
                dq[b, h, r0:r1] = da @ k[b, h, :r1]
                dk[b, h, :r1] += da.T @ q[b, h, r0:r1]
                dv[b, h, :r1] += scale * (a.T @ do[b, h, r0:r1])
    return dq, dk, dv


def linear_pairs(N: int, B: int = 1, H: int = 1) -> int:
    """Visible (query, key) pairs of the causal mask over B*H heads."""
    return B * H * N * (N + 1) // 2
