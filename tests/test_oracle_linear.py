"""Pins for the causal linear-attention oracle (oracle/linear.py), CPU only.

Pages: "Lightning Attention-2: A Free Lunch for Handling Unlimited Sequence
Lengths in Large Language Models" (abstract: intra-block attention-style
computation, inter-block kernel trick) and "[Paper review] Gated Linear
Attention Transformers with Hardware-Efficient Training" (abstract: linear
attention as an RNN with a matrix-valued hidden state; "proposed method":
chunkwise form, recurrence between chunks, parallel inside a chunk).

The oracle is the quadratic definition O = scale * tril(Q K^T) V.  It is
pinned by forms computed differently: exactly rounded brute force, the
recurrent form with a d x d state, the chunkwise intra/inter split with
ragged chunks, closed forms (N = 1; prefix sums when every score is 1),
linearity; plus planted mistakes.  The backward oracle (the analytic
gradient of <dO, O>) is pinned by central finite differences, reverse mode
through the recurrent form, torch.autograd in float64, the N = 1 closed
form and the chunkwise backward with ragged chunks.
"""
import math
import types

import numpy as np
import pytest

import oracle.linear as OL


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def _close(a, b, tol, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, (what, err, tol)


def pin_bruteforce(m):
    """Explicit loops with exactly rounded sums (math.fsum)."""
    for N, d, dv in ((1, 1, 1), (2, 3, 2), (5, 2, 3), (9, 4, 4)):
        q, k, v = _rand(1, 1, 1, N, d), _rand(2, 1, 1, N, d), _rand(3, 1, 1, N, dv)
        o = m.linear_attention_fwd(q, k, v, 0.7)
        ref = np.zeros((N, dv))
        for i in range(N):
            for c in range(dv):
                ref[i, c] = 0.7 * math.fsum(
                    math.fsum(q[0, 0, i, t] * k[0, 0, j, t] for t in range(d))
                    * v[0, 0, j, c] for j in range(i + 1))
        _close(o[0, 0], ref, 1e-12, f"brute N={N}")


def pin_recurrent(m):
    """The RNN form: S_i = S_{i-1} + k_i^T v_i (d x d), o_i = scale q_i S_i."""
    B, H, N, d = 2, 2, 37, 8
    q, k, v = _rand(4, B, H, N, d), _rand(5, B, H, N, d), _rand(6, B, H, N, d)
    o = m.linear_attention_fwd(q, k, v, 0.25)
    ref = np.zeros_like(o)
    for b in range(B):
        for h in range(H):
            S = np.zeros((d, d))
            for i in range(N):
                S += np.outer(k[b, h, i], v[b, h, i])
                ref[b, h, i] = 0.25 * (q[b, h, i] @ S)
    _close(o, ref, 1e-12, "recurrent")


def _chunkwise(q, k, v, scale, C):
    """Intra-chunk tril(Q_t K_t^T) V_t plus inter-chunk Q_t S_{t-1}."""
    B, H, N, d = q.shape
    o = np.zeros((B, H, N, v.shape[-1]))
    for b in range(B):
        for h in range(H):
            S = np.zeros((d, v.shape[-1]))
            for c0 in range(0, N, C):
                c1 = min(N, c0 + C)
                qt, kt, vt = q[b, h, c0:c1], k[b, h, c0:c1], v[b, h, c0:c1]
                intra = np.tril(qt @ kt.T) @ vt
                o[b, h, c0:c1] = scale * (intra + qt @ S)
                S = S + kt.T @ vt
    return o


def pin_chunkwise(m):
    """The block split of the pages with ragged chunks equals the oracle."""
    B, H, N, d = 1, 3, 50, 6
    q, k, v = _rand(7, B, H, N, d), _rand(8, B, H, N, d), _rand(9, B, H, N, d)
    o = m.linear_attention_fwd(q, k, v, 1.3, row_chunk=16)
    for C in (1, 3, 7, 16, 64):
        _close(o, _chunkwise(q, k, v, 1.3, C), 1e-11, f"chunk {C}")


def pin_closed_forms(m):
    """N = 1: o = scale (q . k) v.  Every score 1 (k_j = e_0, q_i0 = 1):
    o_i = scale * sum_{j <= i} v_j (a prefix sum)."""
    q, k, v = _rand(10, 1, 1, 1, 5), _rand(11, 1, 1, 1, 5), _rand(12, 1, 1, 1, 3)
    o = m.linear_attention_fwd(q, k, v, 0.5)
    _close(o[0, 0, 0], 0.5 * float(q[0, 0, 0] @ k[0, 0, 0]) * v[0, 0, 0], 1e-14)
    N = 23
    q = np.zeros((1, 1, N, 4)); q[..., 0] = 1.0
    k = np.zeros((1, 1, N, 4)); k[..., 0] = 1.0
    v = _rand(13, 1, 1, N, 3)
    o = m.linear_attention_fwd(q, k, v, 2.0, row_chunk=5)
    _close(o[0, 0], 2.0 * np.cumsum(v[0, 0], axis=0), 1e-12, "prefix sums")


def pin_row_subset(m):
    """Rows computed alone equal the same rows of the full computation."""
    B, H, N, d = 1, 2, 40, 5
    q, k, v = _rand(18, B, H, N, d), _rand(19, B, H, N, d), _rand(20, B, H, N, d)
    full = m.linear_attention_fwd(q, k, v, 0.6)
    rows = np.array([0, 3, 17, 39])
    _close(m.linear_attention_fwd(q, k, v, 0.6, rows=rows), full[:, :, rows],
           1e-12, "row subset")


def pin_linearity(m):
    """Linear in V and in Q; homogeneous of degree 1 in K."""
    B, H, N, d = 1, 1, 20, 4
    q, k = _rand(14, B, H, N, d), _rand(15, B, H, N, d)
    v1, v2 = _rand(16, B, H, N, d), _rand(17, B, H, N, d)
    f = lambda q_, k_, v_: m.linear_attention_fwd(q_, k_, v_, 0.9)
    _close(f(q, k, 2 * v1 - 3 * v2), 2 * f(q, k, v1) - 3 * f(q, k, v2), 1e-12)
    _close(f(-1.5 * q, k, v1), -1.5 * f(q, k, v1), 1e-12)
    _close(f(q, 4 * k, v1), 4 * f(q, k, v1), 1e-12)


# ---- backward pins: the gradient of <dO, O> computed other ways.

def _loss(m, q, k, v, do, scale):
    return float(np.sum(do * m.linear_attention_fwd(q, k, v, scale)))


def pin_bwd_finite_differences(m):
    """Central differences of <dO, O> (a cubic polynomial of the inputs,
    so the O(h^2) truncation is ~1e-12 relative) on every input element."""
    B, H, N, d = 1, 2, 7, 3
    q, k, v, do = (_rand(s_, B, H, N, d) for s_ in (30, 31, 32, 33))
    g = m.linear_attention_bwd(q, k, v, do, 0.8)
    h = 1e-5
    for x, gx, name in ((q, g[0], "dQ"), (k, g[1], "dK"), (v, g[2], "dV")):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            x0 = x[idx]
            x[idx] = x0 + h
            lp = _loss(m, q, k, v, do, 0.8)
            x[idx] = x0 - h
            lm = _loss(m, q, k, v, do, 0.8)
            x[idx] = x0
            num[idx] = (lp - lm) / (2 * h)
        _close(gx, num, 1e-8 * max(1.0, float(np.abs(num).max())), name)


def pin_bwd_recurrent(m):
    """Reverse mode through the RNN form (state S_i = sum_{j<=i} k_j^T v_j,
    o_i = scale q_i S_i): dq_i = scale dO_i S_i^T; with
    G_j = scale sum_{t>=j} q_t^T dO_t (a reverse running sum),
    dk_j = v_j G_j^T and dv_j = k_j G_j."""
    B, H, N, d = 2, 2, 29, 6
    q, k, v, do = (_rand(s_, B, H, N, d) for s_ in (34, 35, 36, 37))
    dq, dk, dv = m.linear_attention_bwd(q, k, v, do, 0.45, row_chunk=8)
    rq, rk, rv = (np.zeros_like(q) for _ in range(3))
    for b in range(B):
        for h in range(H):
            S = np.zeros((d, d))
            for i in range(N):
                S += np.outer(k[b, h, i], v[b, h, i])
                rq[b, h, i] = 0.45 * (do[b, h, i] @ S.T)
            G = np.zeros((d, d))
            for j in range(N - 1, -1, -1):
                G += 0.45 * np.outer(q[b, h, j], do[b, h, j])
                rk[b, h, j] = v[b, h, j] @ G.T
                rv[b, h, j] = k[b, h, j] @ G
    _close(dq, rq, 1e-11, "dQ recurrent")
    _close(dk, rk, 1e-11, "dK recurrent")
    _close(dv, rv, 1e-11, "dV recurrent")


def pin_bwd_autograd(m):
    """torch.autograd in float64 on the CPU, on tril(Q K^T) V."""
    import torch
    B, H, N, d = 1, 3, 40, 5
    q, k, v, do = (_rand(s_, B, H, N, d) for s_ in (38, 39, 40, 41))
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True)
                  for x in (q, k, v))
    o = -1.3 * (torch.tril(tq @ tk.transpose(-1, -2)) @ tv)
    (o * torch.tensor(do)).sum().backward()
    g = m.linear_attention_bwd(q, k, v, do, -1.3, row_chunk=16)
    for gx, t, name in zip(g, (tq, tk, tv), ("dQ", "dK", "dV")):
        _close(gx, t.grad.numpy(), 1e-11, name + " autograd")


def pin_bwd_closed_forms(m):
    """N = 1: o = scale (q . k) v, so dq = scale (dO . v) k,
    dk = scale (dO . v) q, dv = scale (q . k) dO."""
    q, k, v, do = (_rand(s_, 1, 1, 1, 4) for s_ in (42, 43, 44, 45))
    dq, dk, dv = m.linear_attention_bwd(q, k, v, do, 0.3)
    qq, kk, vv, gg = q[0, 0, 0], k[0, 0, 0], v[0, 0, 0], do[0, 0, 0]
    _close(dq[0, 0, 0], 0.3 * (gg @ vv) * kk, 1e-14, "dq N=1")
    _close(dk[0, 0, 0], 0.3 * (gg @ vv) * qq, 1e-14, "dk N=1")
    _close(dv[0, 0, 0], 0.3 * (qq @ kk) * gg, 1e-14, "dv N=1")


def _chunk_bwd(q, k, v, do, scale, C):
    """The chunkwise backward: dQ by the causal chunk form of (dO, V, K);
    dK and dV by the same form walked from the last chunk to the first,
    the state G = sum over later chunks of Q_u^T dO_u."""
    B, H, N, d = q.shape
    dq, dk, dv = (np.zeros_like(q) for _ in range(3))
    for b in range(B):
        for h in range(H):
            S = np.zeros((d, d))
            for c0 in range(0, N, C):
                c1 = min(N, c0 + C)
                g, vt, kt = do[b, h, c0:c1], v[b, h, c0:c1], k[b, h, c0:c1]
                dq[b, h, c0:c1] = scale * (np.tril(g @ vt.T) @ kt + g @ S)
                S = S + vt.T @ kt
            G = np.zeros((d, d))
            starts = list(range(0, N, C))
            for c0 in reversed(starts):
                c1 = min(N, c0 + C)
                qt, kt, vt, g = (x[b, h, c0:c1] for x in (q, k, v, do))
                dv[b, h, c0:c1] = scale * (np.triu(kt @ qt.T) @ g + kt @ G)
                dk[b, h, c0:c1] = scale * (np.triu(vt @ g.T) @ qt + vt @ G.T)
                G = G + qt.T @ g
    return dq, dk, dv


def pin_bwd_chunkwise(m):
    """The chunk split the kernels use, with ragged chunks, equals the
    oracle; so does the oracle's own row chunking."""
    B, H, N, d = 1, 2, 45, 7
    q, k, v, do = (_rand(s_, B, H, N, d) for s_ in (46, 47, 48, 49))
    ref = m.linear_attention_bwd(q, k, v, do, 0.6)
    for C in (1, 4, 16, 64):
        for a, b_, name in zip(ref, _chunk_bwd(q, k, v, do, 0.6, C),
                               ("dQ", "dK", "dV")):
            _close(a, b_, 1e-11, f"{name} chunk {C}")
    for rc in (1, 6, 13):
        for a, b_, name in zip(ref, m.linear_attention_bwd(q, k, v, do, 0.6,
                                                           row_chunk=rc),
                               ("dQ", "dK", "dV")):
            _close(a, b_, 1e-11, f"{name} row chunk {rc}")


PINS = [pin_bruteforce, pin_recurrent, pin_chunkwise, pin_closed_forms,
        pin_row_subset, pin_linearity, pin_bwd_finite_differences,
        pin_bwd_recurrent, pin_bwd_autograd, pin_bwd_closed_forms,
        pin_bwd_chunkwise]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_linear_oracle_pin(pin):
    pin(OL)


def test_linear_pairs():
    assert OL.linear_pairs(4096, 4, 16) == 4 * 16 * 4096 * 4097 // 2
    assert OL.linear_pairs(1) == 1


MUTANTS = [
    ("strict_mask", "a = np.where(j <= i, a, 0.0)", "a = np.where(j < i, a, 0.0)"),
    ("reversed_mask", "a = np.where(j <= i, a, 0.0)", "a = np.where(j >= i, a, 0.0)"),
    ("no_mask", "a = np.where(j <= i, a, 0.0)", "a = a"),
    ("no_scale", "o[b, h, r0:r1] = scale * (a @ v[b, h, :n1])",
     "o[b, h, r0:r1] = (a @ v[b, h, :n1])"),
    ("keys_from_q", "a = q[b, h, rr] @ k[b, h, :n1].T",
     "a = q[b, h, rr] @ q[b, h, :n1].T"),
    ("chunk_local_keys", "a = q[b, h, rr] @ k[b, h, :n1].T",
     "a = q[b, h, rr] @ np.concatenate([np.zeros_like(k[b, h, :rr[0]]), k[b, h, rr[0]:n1]]).T"),
    # backward
    ("bwd_strict_mask", "vis = j <= i  ", "vis = j < i  "),
    ("bwd_unmasked_da", "da = np.where(vis, scale", "da = np.where(True, scale"),
    ("bwd_dq_uses_v", "dq[b, h, r0:r1] = da @ k[b, h, :r1]",
     "dq[b, h, r0:r1] = da @ v[b, h, :r1]"),
    ("bwd_dk_uses_k", "dk[b, h, :r1] += da.T @ q[b, h, r0:r1]",
     "dk[b, h, :r1] += da.T @ k[b, h, r0:r1]"),
    ("bwd_dv_no_scale", "dv[b, h, :r1] += scale * (a.T @ do[b, h, r0:r1])",
     "dv[b, h, :r1] += (a.T @ do[b, h, r0:r1])"),
    ("bwd_dv_overwrites", "dv[b, h, :r1] += scale", "dv[b, h, :r1] = scale"),
    ("bwd_da_transposed", "scale * (do[b, h, r0:r1] @ v[b, h, :r1].T)",
     "scale * (v[b, h, r0:r1] @ do[b, h, :r1].T)"),
    ("bwd_dk_from_a", "dk[b, h, :r1] += da.T @ q[b, h, r0:r1]",
     "dk[b, h, :r1] += scale * a.T @ q[b, h, r0:r1]"),
]


def _mutant(old, new):
    with open(OL.__file__) as f:
        src = f.read()
    assert src.count(old) >= 1, old
    mod = types.ModuleType("oracle_linear_mutant")
    exec(compile(src.replace(old, new), "oracle_linear_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[x[0] for x in MUTANTS])
def test_planted_mistake_is_caught(name, old, new):
    mod = _mutant(old, new)
    for pin in PINS:
        try:
            pin(mod)
        except Exception:
            return
    pytest.fail(f"no pin caught the planted mistake {name}")
