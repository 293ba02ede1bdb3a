"""GPU parity of causal linear attention (fa_linear_fwd) against the fp64
oracle O = scale * tril(Q K^T) V (oracle/linear.py).

Pages: "Lightning Attention-2: A Free Lunch for Handling Unlimited Sequence
Lengths in Large Language Models" (abstract) and "[Paper review] Gated
Linear Attention Transformers with Hardware-Efficient Training" (chunkwise
form).

Tolerance, per element, derived from what the kernel rounds (everything
else is float32 accumulation of bf16 products):
  * the intra-chunk scores A = Q_t K_t^T are rounded to bf16 before A V:
    2^-9 relative each, so at most 2^-9 scale sum_j |a_ij| |v_jc| over the
    chunk's keys;
  * the state S_{t-1} (float32) is rounded to bf16 before Q_t S_{t-1}:
    at most 2^-9 scale sum_c' |q_ic'| |S_c'c|;
  * O is rounded to bf16 once: 2^-9 |o| (taken as 2^-8);
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
    q, k, v = (to_dev(inp, n) for n in ("q", "k", "v"))
    o = torch.full_like(q, float("nan"))
    n = fa.fa_linear_workspace_size(*q.shape)
    ws = torch.full((n,), 0x7F, dtype=torch.uint8, device=DEV) if n else None
    fa.fa_linear_fwd(q, k, v, o, inp["scale"], ws)
    torch.cuda.synchronize()
    return o


def _bound(q, k, v, scale, rows):
    """Per-element tolerance for query rows `rows` of one head (q,k,v [N,d])."""
    N = q.shape[0]
    rows = np.asarray(rows)
    a = np.abs(q[rows] @ k.T)                               # |q_i . k_j|
    j = np.arange(N)[None, :]
    i = rows[:, None]
    c0 = (rows // CHUNK * CHUNK)[:, None]
    intra = np.where((j <= i) & (j >= c0), a, 0.0) @ np.abs(v)
    allv = np.where(j <= i, a, 0.0) @ np.abs(v)
    # S_{t-1} = K[:64t]^T V[:64t] for the chunk t of each row (prefix sums
    # over chunks).
    nch = (int(rows.max()) // CHUNK) + 1
    states = np.zeros((nch, k.shape[1], v.shape[1]))
    for t in range(1, nch):
        c = slice((t - 1) * CHUNK, t * CHUNK)
        states[t] = states[t - 1] + k[c].T @ v[c]
    inter = np.stack([np.abs(q[r]) @ np.abs(states[r // CHUNK]) for r in rows])
    o = scale * (np.where(j <= i, q[rows] @ k.T, 0.0) @ v)
    s = abs(scale)
    return (2 * 2.0 ** -9 * s * (intra + inter) + 2.0 ** -8 * np.abs(o)
            + 2.0 ** -20 * s * (allv + inter) + 1e-6)


def _check(name, inp, rows=None, heads=None):
    o = _run(inp)
    og = host64(o)
    q, k, v = inp["q"], inp["k"], inp["v"]
    B, H, N, d = q.shape
    rows = np.arange(N) if rows is None else np.asarray(rows)
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    worst, worst_ratio = 0.0, 0.0
    for b, h in heads:
        qh, kh, vh = (x[b, h].astype(np.float64) for x in (q, k, v))
        ref = OL.linear_attention_fwd(qh[None, None], kh[None, None],
                                      vh[None, None], inp["scale"],
                                      rows=rows)[0, 0]
        tol = _bound(qh, kh, vh, inp["scale"], rows)
        err = np.abs(og[b, h, rows] - ref)
        assert np.all(np.isfinite(og[b, h, rows])), name
        worst = max(worst, float(err.max()))
        worst_ratio = max(worst_ratio, float((err / tol).max()))
        assert np.all(err <= tol), (name, (b, h), float((err / tol).max()))
    report(name, O_max=worst, O_over_bound=worst_ratio)


# Few heads split each sequence into segments (a first pass writes the
# segments' states): (1,1,1000,64), (1,2,2000,128), (1,3,1100,64) and the
# N = 23400 case below; the others run unsplit.
CASES = [(1, 1, 1, 64), (1, 2, 64, 128), (2, 3, 100, 128), (1, 2, 300, 64),
         (3, 4, 513, 64), (2, 5, 1000, 128), (1, 9, 130, 128), (1, 1, 1000, 64),
         (1, 2, 2000, 128), (1, 3, 1100, 64)]


@pytest.mark.parametrize("B,H,N,d", CASES)
def test_linear_small(B, H, N, d):
    inp = S.make_case(B, H, N, d, causal=True, seed=950 + N + d)
    _check(f"linear B{B} H{H} N{N} d{d}", inp)


@pytest.mark.parametrize("scale", [1.0, -0.5, 0.0])
def test_linear_scale(scale):
    inp = S.make_case(1, 2, 200, 128, causal=True, seed=77, scale=scale)
    _check(f"linear scale {scale}", inp)


def test_linear_large_magnitudes():
    inp = S.make_case(1, 2, 700, 64, causal=True, seed=78, q_scale=30.0)
    _check("linear |Q| x30", inp)


def test_linear_long_sequence():
    """A long head (N = 23400, the trading-day length, d = 64): sampled rows
    across the sequence, the state carried over 366 chunks."""
    inp = S.make_case(1, 2, 23400, 64, causal=True, seed=79)
    rows = np.unique(np.concatenate([np.arange(0, 70), np.arange(23330, 23400),
                                     np.random.default_rng(2).integers(0, 23400, 100)]))
    _check("linear N=23400", inp, rows=rows)


def test_linear_split_matches_definition_boundaries():
    """Rows on both sides of every segment boundary of a split sequence."""
    import io_aware_tiled_amd as fa
    N = 3000
    assert fa.fa_linear_workspace_size(1, 1, N, 128) > 0
    inp = S.make_case(1, 1, N, 128, causal=True, seed=80)
    rows = np.unique(np.clip(np.concatenate(
        [np.arange(c - 2, c + 2) for c in range(0, N + 64, 64)]), 0, N - 1))
    _check("linear split boundaries", inp, rows=rows)


def test_linear_workload_sampled():
    """Full-size workload (4 x 16 x 4096 x 128) in the launch configuration
    the benchmark times: sampled rows of four heads."""
    inp = S.make_inputs("linear_causal_d128")
    rows = np.unique(np.concatenate([np.arange(0, 70), np.arange(4026, 4096),
                                     np.random.default_rng(3).integers(0, 4096, 60)]))
    _check("linear workload", inp, rows=rows, heads=[(0, 0), (1, 7), (2, 9), (3, 15)])
