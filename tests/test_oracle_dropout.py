"""Pins for the attention-dropout oracle (oracle/dropout.py), CPU only.

Page: "Is a full-day context better than a 10-minute context? Flash
attention and the sequence-length question" (marketmaker.cc blog),
"Integration": the framework call carries a dropout probability.  The
generator is Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
numbers: as easy as 1, 2, 3", SC 2011).

Pinned by: the generator's published known-answer vectors
(tests/golden/philox4x32_10_kat.json); the element -> (counter, word, byte)
mapping against scalar generator calls; keep frequencies within binomial
bounds and uniform bytes; p8 = 0 reducing exactly to the dense oracle;
explicit loops with exactly rounded sums; unbiasedness over many masks;
finite differences of <dO, O> for a fixed mask; plus planted mistakes.
"""
import json
import math
import os
import types

import numpy as np
import pytest

import oracle.attention as OA
import oracle.dropout as OD

GOLDEN = os.path.join(os.path.dirname(__file__), "golden",
                      "philox4x32_10_kat.json")


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def pin_kat(m):
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        ctr = [int(x, 16) for x in c["counter"]]
        key = [int(x, 16) for x in c["key"]]
        out = m.philox4x32_10(*ctr, *key)
        got = [int(np.asarray(w).reshape(-1)[0]) for w in out]
        assert got == [int(x, 16) for x in c["output"]], (c, [hex(g) for g in got])


def pin_mapping(m):
    """keep_mask element (i, j) = byte j%4 of word i%4 of the call at
    counter (j//4, i//4, bh, offset), key (seed low, seed high)."""
    seed, off, bh, p8 = 0x0123456789ABCDEF, 5, 3, 100
    rows = np.array([0, 1, 2, 3, 5, 6, 11, 17, 30])
    n = 23
    z = m.keep_mask(seed, off, p8, bh, rows, n)
    assert z.shape == (len(rows), n)
    for a, i in enumerate(rows):
        for j in range(n):
            words = m.philox4x32_10(j // 4, i // 4, bh, off, seed & 0xFFFFFFFF,
                                    seed >> 32)
            w = int(np.asarray(words[i % 4]).reshape(-1)[0])
            byte = (w >> (8 * (j % 4))) & 0xFF
            assert bool(z[a, j]) == (byte >= p8), (i, j)


def pin_frequencies(m):
    """Keep frequency (256 - p8)/256 within 5 sigma; p8 = 0 keeps all;
    bytes of every (i%4, j%4) position are uniform (chi-square)."""
    rows = np.arange(512)
    assert m.keep_mask(9, 0, 0, 0, rows, 512).all()
    for p8 in (1, 26, 128, 255):
        z = m.keep_mask(11, 1, p8, 2, rows, 512)
        k = (256 - p8) / 256
        sd = math.sqrt(k * (1 - k) / z.size)
        assert abs(z.mean() - k) < 5 * sd + 1e-12, (p8, z.mean(), k)
    # Uniform bytes: counts of byte >= t for t = 64, 128, 192 per position.
    for t in (64, 128, 192):
        z = m.keep_mask(13, 2, t, 1, rows, 512)
        for a in range(4):
            for b in range(4):
                f = z[a::4, b::4].mean()
                k = (256 - t) / 256
                sd = math.sqrt(k * (1 - k) / z[a::4, b::4].size)
                assert abs(f - k) < 5 * sd, (t, a, b, f)
    # Different offsets, seeds and heads give different masks.
    base = m.keep_mask(1, 0, 128, 0, rows[:64], 64)
    for other in (m.keep_mask(1, 1, 128, 0, rows[:64], 64),
                  m.keep_mask(2, 0, 128, 0, rows[:64], 64),
                  m.keep_mask(1, 0, 128, 1, rows[:64], 64)):
        assert 0.3 < (base != other).mean() < 0.7


def pin_no_drop(m):
    """p8 = 0: the dense oracle exactly (forward and backward)."""
    B, H, N, d = 1, 2, 19, 5
    q, k, v, do = (_rand(s, B, H, N, d) for s in (21, 22, 23, 24))
    for causal in (False, True):
        o, lse = m.attention_dropout_fwd(q, k, v, 0.4, causal, 0, 77)
        o2, lse2 = OA.attention_fwd(q, k, v, 0.4, causal)
        assert np.max(np.abs(o - o2)) < 1e-13
        assert np.max(np.abs(lse - lse2)) < 1e-13
        g = m.attention_dropout_bwd(q, k, v, do, 0.4, causal, 0, 77)
        g2 = OA.attention_bwd(q, k, v, do, 0.4, causal)
        for a, b in zip(g, g2):
            assert np.max(np.abs(a - b)) < 1e-12


def pin_bruteforce(m):
    """Explicit loops (math.fsum) with the mask taken element by element."""
    N, d, scale, p8, seed, off = 9, 3, 0.8, 90, 1234, 3
    q, k, v = _rand(31, 1, 1, N, d), _rand(32, 1, 1, N, d), _rand(33, 1, 1, N, d)
    for causal in (False, True):
        o, lse = m.attention_dropout_fwd(q, k, v, scale, causal, p8, seed, off)
        z = m.keep_mask(seed, off, p8, 0, np.arange(N), N)
        kp = (256 - p8) / 256
        for i in range(N):
            keys = range(i + 1) if causal else range(N)
            s = [scale * math.fsum(q[0, 0, i, t] * k[0, 0, j, t] for t in range(d))
                 for j in keys]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            l = math.fsum(e)
            assert abs(lse[0, 0, i] - (mx + math.log(l))) < 1e-12
            for c in range(d):
                ref = math.fsum(e[a] / l * (1.0 if z[i, j] else 0.0) / kp * v[0, 0, j, c]
                                for a, j in enumerate(keys))
                assert abs(o[0, 0, i, c] - ref) < 1e-12, (causal, i, c)


def pin_unbiased(m):
    """The mean over many masks (offsets) approaches the dense output,
    within 6 standard errors per element."""
    B, H, N, d = 1, 1, 12, 3
    q, k, v = _rand(41, B, H, N, d), _rand(42, B, H, N, d), _rand(43, B, H, N, d)
    p8, T = 77, 600
    kp = (256 - p8) / 256
    dense, _ = OA.attention_fwd(q, k, v, 0.5, True)
    acc = np.zeros_like(dense)
    for t in range(T):
        acc += m.attention_dropout_fwd(q, k, v, 0.5, True, p8, 99, t)[0]
    mean = acc / T
    P = OA.attention_probs(q, k, 0.5, True)[0, 0]
    var = (P ** 2) @ (v[0, 0] ** 2) * (1 - kp) / kp
    se = np.sqrt(var / T)
    assert np.all(np.abs(mean[0, 0] - dense[0, 0]) <= 6 * se + 1e-12)


def pin_finite_differences(m):
    """dQ, dK, dV against central differences of L = <dO, O> with the mask
    fixed (it does not depend on Q, K, V)."""
    B, H, N, d = 1, 2, 7, 3
    q, k, v, do = (_rand(s, B, H, N, d) for s in (51, 52, 53, 54))
    args = (0.7, True, 64, 4242, 1)
    dq, dk, dv = m.attention_dropout_bwd(q, k, v, do, *args)
    L = lambda q_, k_, v_: float(np.sum(do * m.attention_dropout_fwd(q_, k_, v_, *args)[0]))
    h = 1e-6
    for x, g, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        for idx in [(0, 0, 0, 0), (0, 1, 3, 2), (0, 1, 6, 1), (0, 0, 4, 0)]:
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            ins_p = [q, k, v]
            ins_m = [q, k, v]
            ins_p[which], ins_m[which] = xp, xm
            fd = (L(*ins_p) - L(*ins_m)) / (2 * h)
            assert abs(fd - g[idx]) < 1e-6 * max(1.0, abs(fd)), (which, idx, fd, g[idx])


PINS = [pin_kat, pin_mapping, pin_frequencies, pin_no_drop, pin_bruteforce,
        pin_unbiased, pin_finite_differences]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_dropout_oracle_pin(pin):
    pin(OD)


MUTANTS = [
    ("multiplier", "_M0 = np.uint64(0xD2511F53)", "_M0 = np.uint64(0xD2511F55)"),
    ("weyl", "_W1 = 0xBB67AE85", "_W1 = 0xBB67AE87"),
    ("nine_rounds", "for _ in range(10):", "for _ in range(9):"),
    ("word_from_key", "word = w[(rows % 4)[:, None],", "word = w[kb % 4,"),
    ("byte_order", "byte = (word[:, :, None] >> shifts)", "byte = (word[:, :, None] >> shifts[::-1])"),
    ("counter_swap", "philox4x32_10(kb, qb,", "philox4x32_10(qb, kb,"),
    ("strict_threshold", "return (byte >= np.uint32(p8))", "return (byte > np.uint32(p8))"),
    ("no_rescale", "o[b, h] = (p * z / kp) @ v[b, h]", "o[b, h] = (p * z) @ v[b, h]"),
    ("bwd_dp_unmasked", "dp = (do[b, h] @ v[b, h].T) * z / kp", "dp = (do[b, h] @ v[b, h].T) / kp"),
    ("bwd_dv_unscaled", "dv[b, h] = (p * z / kp).T @ do[b, h]", "dv[b, h] = (p * z).T @ do[b, h]"),
]


def _mutant(old, new):
    with open(OD.__file__) as f:
        src = f.read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle_dropout_mutant")
    exec(compile(src.replace(old, new), "oracle_dropout_mutant", "exec"), mod.__dict__)
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
