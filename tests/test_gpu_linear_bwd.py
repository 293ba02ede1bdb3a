"""GPU parity of the causal linear-attention backward (fa_linear_bwd)
against the fp64 oracle's analytic gradients (oracle/linear.py).

Pages: "Lightning Attention-2: A Free Lunch for Handling Unlimited Sequence
Lengths in Large Language Models" (abstract: the tiled forward and backward)
and "[Paper review] Gated Linear Attention Transformers with
Hardware-Efficient Training" (chunkwise form for training).

Each gradient is one chunkwise pass out_i = scale * sum_{j in vis(i)}
(a_i . b_j) c_j: dQ with (a, b, c) = (dO, V, K) and vis(i) = {j <= i}; dK
with (V, dO, Q) and dV with (K, Q, dO), both with vis(i) = {j >= i}.  The
tolerance per element is derived from what such a pass rounds, exactly as
for the forward:
  * the intra-chunk scores a_i . b_j are rounded to bf16 before the product
    with c: 2^-9 relative each, at most 2^-9 scale sum_j |a_i . b_j| |c_j|
    over the chunk;
  * the float32 state (sum of b_j^T c_j over the earlier, or later, chunks)
    is rounded to bf16 before a_i S: at most 2^-9 scale sum |a_i| |S|;
  * the output is rounded to bf16 once: 2^-9 |out| (taken as 2^-8);
  * float32 accumulation: 2^-20 of the sum of all product magnitudes.
Both rounding terms are doubled for margin.
"""
import numpy as np
import pytest

import oracle.linear as OL
import synthetic as S
from gpu_util import DEV, host64, report, to_dev

pytestmark = pytest.mark.gpu
CHUNK = 64


def _run(inp):
    import torch
    import io_aware_tiled_amd as fa
    q, k, v, do = (to_dev(inp, n) for n in ("q", "k", "v", "do"))
    outs = [torch.full_like(q, float("nan")) for _ in range(3)]
    n = fa.fa_linear_workspace_size(*q.shape)
    ws = torch.full((n,), 0x7F, dtype=torch.uint8, device=DEV) if n else None
    fa.fa_linear_bwd(q, k, v, do, *outs, inp["scale"], ws)
    torch.cuda.synchronize()
    return outs


def _bound(a, b, c, scale, rev):
    """Per-element tolerance of one pass over one head (a, b, c [N, d])."""
    N = a.shape[0]
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    vis = (j >= i) if rev else (j <= i)
    same = (i // CHUNK) == (j // CHUNK)
    ab = np.abs(a @ b.T)
    intra = np.where(vis & same, ab, 0.0) @ np.abs(c)
    allv = np.where(vis, ab, 0.0) @ np.abs(c)
    nch = (N + CHUNK - 1) // CHUNK
    per = np.stack([b[t * CHUNK:(t + 1) * CHUNK].T @ c[t * CHUNK:(t + 1) * CHUNK]
                    for t in range(nch)])                  # chunk states
    if rev:
        st = np.cumsum(per[::-1], axis=0)[::-1]            # chunks >= t
        st = np.concatenate([st[1:], np.zeros_like(st[:1])])   # chunks > t
    else:
        st = np.cumsum(per, axis=0)                        # chunks <= t
        st = np.concatenate([np.zeros_like(st[:1]), st[:-1]])  # chunks < t
    inter = np.stack([np.abs(a[r]) @ np.abs(st[r // CHUNK]) for r in range(N)])
    out = scale * (np.where(vis, a @ b.T, 0.0) @ c)
    s = abs(scale)
    return (2 * 2.0 ** -9 * s * (intra + inter) + 2.0 ** -8 * np.abs(out)
            + 2.0 ** -20 * s * (allv + inter) + 1e-6)


def _check(name, inp, heads=None):
    dq, dk, dv = (host64(t) for t in _run(inp))
    q, k, v, do = (inp[n].astype(np.float64) for n in ("q", "k", "v", "do"))
    B, H, N, d = q.shape
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    worst = {"dQ": 0.0, "dK": 0.0, "dV": 0.0}
    ratio = dict(worst)
    sc = inp["scale"]
    for b, h in heads:
        sel = lambda x: x[b, h][None, None]
        ref = OL.linear_attention_bwd(sel(q), sel(k), sel(v), sel(do), sc)
        passes = {"dQ": (do[b, h], v[b, h], k[b, h], False, dq[b, h]),
                  "dK": (v[b, h], do[b, h], q[b, h], True, dk[b, h]),
                  "dV": (k[b, h], q[b, h], do[b, h], True, dv[b, h])}
        for (nm, (a_, b_, c_, rev, got)), r in zip(passes.items(), ref):
            assert np.all(np.isfinite(got)), (name, nm)
            tol = _bound(a_, b_, c_, sc, rev)
            err = np.abs(got - r[0, 0])
            worst[nm] = max(worst[nm], float(err.max()))
            ratio[nm] = max(ratio[nm], float((err / tol).max()))
            assert np.all(err <= tol), (name, nm, (b, h), float((err / tol).max()))
    report(name, **worst, **{k_ + "_over_bound": v_ for k_, v_ in ratio.items()})


# Few heads split each sequence into segments (a first pass writes the
# segments' states, which the reversed passes sum from the later segments):
# (1,1,1000,64), (1,2,2000,128), (1,3,1100,64); the others run unsplit.
CASES = [(1, 1, 1, 64), (1, 2, 64, 128), (2, 3, 100, 128), (1, 2, 300, 64),
         (3, 4, 513, 64), (2, 5, 1000, 128), (1, 9, 130, 128), (1, 1, 1000, 64),
         (1, 2, 2000, 128), (1, 3, 1100, 64)]


@pytest.mark.parametrize("B,H,N,d", CASES)
def test_linear_bwd_small(B, H, N, d):
    inp = S.make_case(B, H, N, d, causal=True, seed=960 + N + d, backward=True)
    _check(f"linear bwd B{B} H{H} N{N} d{d}", inp)


@pytest.mark.parametrize("scale", [1.0, -0.5, 0.0])
def test_linear_bwd_scale(scale):
    inp = S.make_case(1, 2, 200, 128, causal=True, seed=97, scale=scale,
                      backward=True)
    _check(f"linear bwd scale {scale}", inp)


def test_linear_bwd_split_boundaries():
    """A split sequence (N = 3000, one head): every row, so both sides of
    every segment boundary, for all three gradients."""
    import io_aware_tiled_amd as fa
    assert fa.fa_linear_workspace_size(1, 1, 3000, 128) > 0
    inp = S.make_case(1, 1, 3000, 128, causal=True, seed=98, backward=True)
    _check("linear bwd split", inp)


def test_linear_bwd_workload_heads():
    """Full-size workload (4 x 16 x 4096 x 128) in the launch configuration
    the benchmark times: four heads (one per batch entry), every row."""
    inp = S.make_inputs("linear_causal_fwd_bwd_d128")
    _check("linear bwd workload", inp, heads=[(0, 0), (1, 7), (2, 9), (3, 15)])
