"""fp64 CPU oracle for exact scaled-dot-product attention, forward and backward.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The product path (the HIP library
and its Python binding) never imports, calls or links it, and this package
imports nothing from the product path: the two share no code.

Pages cited (titles as given on the pages):
  [MM] "Is a full-day context better than a 10-minute context? Flash attention
       and the sequence-length question" (marketmaker.cc blog)
  [ZN] "Paper summary: FlashAttention" (zenn.dev)
  [TW] "Flash-Attention 2 for performance optimisation" (Medium blog)

What it computes.  The plain definition softmax(scale * Q K^T) V
([MM] "Why attention is memory-bound"; [TW] "Attention": each row of the
attention distribution is a probability distribution summing to one).  The
pages say FlashAttention returns exactly this result, not an approximation
([ZN] "Overview"; [MM] "Online softmax recurrence": the recurrence is a
reassociation of the two-pass softmax).  So the oracle is the definition
itself, evaluated as a two-pass row softmax in float64: pass 1 takes the row
maximum, pass 2 exponentiates, sums and normalises.  Rows are processed in
chunks; each row is computed whole, so chunking is only a memory bound and
never rescales anything across chunks.

Readings where the pages are silent (each also listed in the design notes):
  * `scale` is a parameter; the workloads use 1/sqrt(d) rounded to float32.
  * Masks: key j is visible to query i iff (not causal or j <= i) and
    j < kv_len[b].  Causal alignment is top-left with the diagonal visible
    ([MM] "Causal masking" and the masked_fill(-inf) code of "Integration").
  * The stored statistic is the natural-log log-sum-exp LSE_i = m_i + ln l_i
    ([TW] "Flash Attention 2": FA2 stores L instead of m and l).
  * A row with no visible key gives O = 0 and LSE = -inf.
  * Block-sparse attention ([ZN] "Overview": block-sparse FlashAttention
    skips whole blocks of the score matrix by a fixed block mask; the page
    gives no further detail) is read as the definition restricted by a
    boolean block mask M [H, ceil(N/bq), ceil(N/bk)]: key j is also required
    to satisfy M[h, i // bq, j // bk] for query i of head h, for every batch
    entry.  bq = 256 query rows and bk = 128 keys unless given.
  * Backward: the pages give no formulas, only that P is recomputed from the
    stored statistics ([MM] "Backward pass: recompute instead of store";
    [TW] "Recomputation").  The oracle is the analytic gradient of
    <dO, O> with respect to Q, K, V:
        dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij,
        dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
    It recomputes P with the forward's own definition.

Every input is converted to float64; callers pass the exact values the GPU
sees (bf16- or fp32-rounded), and scale as float64(float32(scale)).
"""
from __future__ import annotations

import concurrent.futures as _cf

import numpy as np

__all__ = ["attention_fwd", "attention_bwd", "attention_probs",
           "visible_mask", "visible_pairs"]


def visible_mask(r0: int, r1: int, n_keys: int, causal: bool,
                 kv_len_b: int | None, rows: np.ndarray | None = None,
                 block_mask: np.ndarray | None = None, bq: int = 256,
                 bk: int = 128) -> np.ndarray:
    """Boolean [rows, n_keys]: True where key j is visible to query i.

    Query indices are r0..r1-1, or `rows` when given.  block_mask: optional
    boolean [ceil(N/bq), ceil(N/bk)] of one head.
    """
    i = (np.arange(r0, r1) if rows is None else np.asarray(rows))[:, None]
    j = np.arange(n_keys)[None, :]
    vis = np.ones((i.shape[0], n_keys), dtype=bool)
    if kv_len_b is not None:
        vis &= j < int(kv_len_b)
    if causal:
        vis &= j <= i
    if block_mask is not None:
        vis &= np.asarray(block_mask, dtype=bool)[i // bq, j // bk]
    return vis


def visible_pairs(N: int, causal: bool, kv_len=None, B: int = 1,
                  H: int = 1) -> int:
    """Number of visible (query, key) pairs over all B*H heads."""
    total = 0
    for b in range(B):
        L = N if kv_len is None else max(0, min(int(kv_len[b]), N))
        if causal:
            # rows i see keys 0..min(i, L-1)
            per = sum(min(i + 1, L) for i in range(N))
        else:
            per = N * L
        total += per * H
    return total


def _probs_rows(qh, kh, scale, causal, kv_len_b, r0, r1, rows=None,
                bmask=None, bq=256, bk=128):
    """Two-pass softmax of one head's query rows.

    Returns (P [rows, N], m [rows], l [rows]); for rows without a visible
    key P is all zero, m = -inf and l = 0.
    """
    qr = qh[r0:r1] if rows is None else qh[rows]
    s = scale * (qr @ kh.T)                              # fp64 scores
    vis = visible_mask(r0, r1, kh.shape[0], causal, kv_len_b, rows,
                       bmask, bq, bk)
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)                                    # pass 1: row max
    empty = ~np.isfinite(m)
    m_ref = np.where(empty, 0.0, m)                      # avoid inf - inf
    e = np.exp(s - m_ref[:, None])                       # pass 2: exp
    l = e.sum(axis=1)
    p = e / np.where(empty, 1.0, l)[:, None]
    return p, m, l


def _heads(B, H):
    return [(b, h) for b in range(B) for h in range(H)]


def _run(fn, items, workers):
    if workers is None or workers <= 1:
        return [fn(it) for it in items]
    with _cf.ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, items))


def attention_fwd(q, k, v, scale, causal=False, kv_len=None, rows=None,
                  row_chunk=512, workers=None, block_mask=None,
                  block_q=256, block_k=128):
    """O and LSE of softmax(scale * Q K^T) V, float64.

    q, k, v: [B, H, N, d].  kv_len: None or int [B].  rows: optional 1-D
    array of query indices; then only those rows are computed and the
    outputs have that many rows.  workers: optional thread count over
    (b, h) heads (numpy releases the GIL in BLAS and exp).  block_mask:
    optional boolean [H, ceil(N/block_q), ceil(N/block_k)], the block-sparse
    pattern of each head (the same for every batch entry).

    Returns (o [B,H,R,d] float64, lse [B,H,R] float64).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    scale = float(scale)
    B, H, N, d = q.shape
    R = N if rows is None else len(rows)
    o = np.zeros((B, H, R, v.shape[-1]), dtype=np.float64)
    lse = np.empty((B, H, R), dtype=np.float64)

    def one(bh):
        b, h = bh
        L = None if kv_len is None else int(kv_len[b])
        bm = None if block_mask is None else block_mask[h]
        for c0 in range(0, R, row_chunk):
            c1 = min(R, c0 + row_chunk)
            if rows is None:
                p, m, l = _probs_rows(q[b, h], k[b, h], scale, causal, L,
                                      c0, c1, None, bm, block_q, block_k)
            else:
                p, m, l = _probs_rows(q[b, h], k[b, h], scale, causal, L,
                                      0, 0, np.asarray(rows)[c0:c1], bm,
                                      block_q, block_k)
            o[b, h, c0:c1] = p @ v[b, h]
            with np.errstate(divide="ignore"):
                lse[b, h, c0:c1] = np.where(np.isfinite(m),
                                            m + np.log(np.where(l > 0, l, 1)),
                                            -np.inf)
        return None

    _run(one, _heads(B, H), workers)
    return o, lse


def attention_probs(q, k, scale, causal=False, kv_len=None):
    """The full attention matrix P [B,H,N,N] (small inputs only)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, H, N, _ = q.shape
    P = np.zeros((B, H, N, k.shape[2]), dtype=np.float64)
    for b, h in _heads(B, H):
        L = None if kv_len is None else int(kv_len[b])
        P[b, h] = _probs_rows(q[b, h], k[b, h], float(scale), causal, L,
                              0, N)[0]
    return P


def attention_bwd(q, k, v, do, scale, causal=False, kv_len=None,
                  row_chunk=512, workers=None, block_mask=None, block_q=256,
                  block_k=128):
    """Analytic gradients (dQ, dK, dV) of <dO, O>, float64, [B,H,N,d] each.

    P is recomputed from Q and K by the forward's definition (with the same
    optional block mask as attention_fwd); D_i is the row sum of P * dP
    (equal to dO_i . O_i).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    scale = float(scale)
    B, H, N, d = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)

    def one(bh):
        b, h = bh
        L = None if kv_len is None else int(kv_len[b])
        bm = None if block_mask is None else block_mask[h]
        for c0 in range(0, N, row_chunk):
            c1 = min(N, c0 + row_chunk)
            p, _, _ = _probs_rows(q[b, h], k[b, h], scale, causal, L, c0, c1,
                                  None, bm, block_q, block_k)
            dor = do[b, h, c0:c1]
            dv[b, h] += p.T @ dor
            dp = dor @ v[b, h].T
            D = (p * dp).sum(axis=1)
            ds = p * (dp - D[:, None])
            dq[b, h, c0:c1] = scale * (ds @ k[b, h])
            dk[b, h] += scale * (ds.T @ q[b, h, c0:c1])
        return None

    _run(one, _heads(B, H), workers)
    return dq, dk, dv
