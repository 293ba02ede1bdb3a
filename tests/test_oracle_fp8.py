"""Pins for the CPU model of the FP8 forward (oracle/fp8.py), CPU only.

Page: "Is a full-day context better than a 10-minute context? Flash attention
and the sequence-length question" (marketmaker.cc), section "FA3: Hopper",
item 3 (random rotation before block-wise FP8 quantisation lowers the error
of FP8 attention on inputs with outliers).

Each pin checks the model against something other than itself: the E4M3
value table of the OCP 8-bit floating-point specification (constants
written out by hand), PyTorch's own float8_e4m3fn conversion, scipy's
Hadamard matrix, brute-force searches, closed forms for one-hot rows,
inputs on which every quantisation step is exact (the model must then equal
the exact oracle), and the page's qualitative claim.  A final test plants
plausible mistakes in a copy of the model and checks a pin catches each.
"""
import types

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle.attention as ORA
import oracle.fp8 as F8
import synthetic as S


def _close(a, b, tol, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, (what, err, tol)


# ---------------------------------------------------------------- pins ----

def pin_e4m3_table(m):
    """Values fixed by the OCP E4M3 definition (bias 7, no infinities)."""
    t = m.e4m3_decode(np.arange(256))
    for code, val in [(0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9),
                      (0x08, 2.0 ** -6), (0x38, 1.0), (0x39, 1.125),
                      (0x40, 2.0), (0x7E, 448.0), (0x77, 240.0),
                      (0x80, -0.0), (0xB8, -1.0), (0xFE, -448.0)]:
        assert t[code] == val and np.signbit(t[code]) == np.signbit(val), hex(code)
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert m.E4M3_MAX == 448.0


def pin_e4m3_torch(m):
    """Library cross-check: torch's float32 -> float8_e4m3fn conversion."""
    rng = np.random.default_rng(5)
    pos = m.e4m3_decode(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2                    # every tie
    near = np.concatenate([np.nextafter(mids.astype(np.float32), np.float32(0)),
                           np.nextafter(mids.astype(np.float32), np.float32(1e9))])
    rand = np.concatenate([
        rng.uniform(0, 448, 4000), np.exp2(rng.uniform(-14, 8.8, 4000)),
        rng.uniform(0, 2.0 ** -6, 2000)])
    x = np.concatenate([mids, near, rand, pos]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    x = np.concatenate([x, -x])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = m.e4m3_encode(x)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (x[bad[:5]], got[bad[:5]], ref[bad[:5]])


def pin_e4m3_roundtrip(m):
    """encode(decode(c)) == c for every finite code; ties go to even."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    assert np.array_equal(m.e4m3_encode(m.e4m3_decode(codes).astype(np.float32)),
                          codes.astype(np.uint8))
    # 1 + 1/16 lies halfway between 1 (0x38, even) and 1.125 (0x39).
    assert m.e4m3_encode(np.float32(1.0625)) == 0x38
    assert m.e4m3_encode(np.float32(1.1875)) == 0x3A   # 1.125 | 1.25 -> even
    assert m.e4m3_encode(np.float32(2.0 ** -10)) == 0x00   # half the least
    assert m.e4m3_encode(np.float32(3 * 2.0 ** -10)) == 0x02


def pin_fwht_scipy(m):
    """The transform is x H_d with scipy's Sylvester-Hadamard matrix (exact
    on small integers), and H_d H_d = d I."""
    rng = np.random.default_rng(7)
    for d in (2, 8, 64, 128):
        x = rng.integers(-50, 50, (5, d)).astype(np.float32)
        Hd = scipy.linalg.hadamard(d).astype(np.float64)
        _close(m.fwht_f32(x), x.astype(np.float64) @ Hd, 0.0, f"fwht {d}")
        _close(m.fwht_f32(m.fwht_f32(x)), d * x, 0.0, "H H = d I")


def pin_rotation_one_hot(m):
    """Signs first, then the transform: row e_i maps to s_i * H_d[i, :]."""
    d = 64
    s = S.rotation_signs(11, d)
    Hd = scipy.linalg.hadamard(d)
    for i in (0, 1, 17, 63):
        e = np.zeros(d, np.float32)
        e[i] = 1.0
        _close(m.rotate_f32(e, s), s[i] * Hd[i], 0.0, f"one-hot {i}")
    # R R^T = d I for the signed map.
    R = np.stack([m.rotate_f32(np.eye(d, dtype=np.float32)[i], s) for i in range(d)])
    _close(R.astype(np.float64) @ R.T, d * np.eye(d), 0.0, "R R^T")


def pin_mx_exponent_bruteforce(m):
    """Smallest e with amax <= 448 2^e, by search, including exact powers,
    the 1.75 mantissa boundary and zero."""
    rng = np.random.default_rng(9)
    a = np.concatenate([
        np.exp2(rng.uniform(-30, 30, 3000)),
        448.0 * np.exp2(np.arange(-20, 20)),                      # boundary
        np.nextafter(448.0 * np.exp2(np.arange(-20, 20)), np.inf),
        np.exp2(np.arange(-20, 20)), 1.75 * np.exp2(np.arange(-5, 5)),
    ]).astype(np.float32).astype(np.float64)
    e = m.mx_exponent(a)
    for ai, ei in zip(a, e):
        want = next(k for k in range(-140, 140) if ai <= 448.0 * 2.0 ** k)
        assert ei == max(want, -127), (ai, ei, want)
    assert m.mx_exponent(np.array([0.0]))[0] == -127


def pin_mx_quantize_bound(m):
    """Dequantised values are within half an E4M3 step of the input: relative
    2^-4 for scaled magnitudes >= 2^-6, absolute 2^-10 * 2^e below; blocks
    are 32 consecutive values of the last axis."""
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((7, 128)) * np.exp2(rng.uniform(-8, 8, (7, 1)))
         ).astype(np.float32)
    x[3, 40] = 5000.0                                  # one large block
    codes, e = m.mx_quantize(x)
    assert codes.shape == x.shape and e.shape == (7, 4)
    assert e[3, 1] > e[3, 0] and e[3, 1] > e[3, 2]     # only block 1 of row 3
    deq = m.mx_dequantize(codes, e)
    eb = np.repeat(e, 32, axis=1).astype(np.float64)
    xs = np.ldexp(np.abs(x.astype(np.float64)), -eb.astype(int))
    bound = np.where(xs >= 2.0 ** -6, xs * 2.0 ** -4, 2.0 ** -10) * np.exp2(eb)
    assert np.all(np.abs(deq - x) <= bound)
    # Each block's largest magnitude uses the top binade of the range.
    amax = np.abs(x.reshape(7, 4, 32)).max(axis=-1)
    assert np.all((amax <= 448.0 * np.exp2(e)) & (amax > 224.0 * np.exp2(e)))


def _exact_case(seed, B, H, N, d):
    """Q, K rows that are +-2^a times a one-hot vector (their rotations are
    +-2^a everywhere) and V of small integers: every quantisation is exact."""
    rng = np.random.default_rng(seed)
    def onehot_rows():
        x = np.zeros((B, H, N, d), np.float32)
        idx = rng.integers(0, d, (B, H, N))
        val = rng.choice([-1.0, 1.0], (B, H, N)) * np.exp2(rng.integers(-3, 3, (B, H, N)))
        np.put_along_axis(x, idx[..., None], val[..., None].astype(np.float32), -1)
        return x
    q, k = onehot_rows(), onehot_rows()
    v = rng.integers(-15, 16, (B, H, N, d)).astype(np.float32)
    return q, k, v


def pin_fp8_exact_reduction(m):
    """When every rotation and quantisation is exact the model equals the
    exact definition (with and without rotation, causal or not)."""
    for d in (64, 128):
        q, k, v = _exact_case(21 + d, 1, 2, 45, d)
        s = S.rotation_signs(3, d)
        for causal in (False, True):
            o_ref, l_ref = ORA.attention_fwd(q, k, v, 0.5, causal)
            for signs in (None, s):
                r = m.fp8_forward(q, k, v, 0.5, causal, signs)
                _close(r["o"], o_ref, 1e-12, f"O d={d} rot={signs is not None}")
                _close(r["lse"], l_ref, 1e-12, "LSE")
                _close(r["q_deq"], q if signs is None else m.rotate_f32(q, s),
                       0.0, "Q exact")


def pin_fp8_layout(m):
    """Shapes and block axes of the quantised operands: Q/K blocks run along
    the head dimension, V blocks along the keys of one channel (keys past N
    are zero)."""
    B, H, N, d = 1, 1, 70, 64
    q, k, v = _exact_case(5, B, H, N, d)
    v[0, 0, 5, 3] = 1000.0
    r = m.fp8_forward(q, k, v, 0.3, False, None)
    assert r["q_codes"].shape == (B, H, N, d) and r["q_exp"].shape == (B, H, N, 2)
    assert r["v_codes"].shape == (B, H, d, 96) and r["v_exp"].shape == (B, H, d, 3)
    ve = r["v_exp"][0, 0]
    assert ve[3, 0] == m.mx_exponent(np.array([1000.0]))[0]
    others = np.ones_like(ve, dtype=bool)
    others[3, 0] = False
    assert ve[3, 0] > ve[others].max()
    assert np.all(r["v_codes"][0, 0, :, 70:] == 0)


def pin_fp8_outlier_claim(m):
    """The page's claim, qualitatively: with outlier features shared by
    queries and keys, the rotated model's error against exact attention is
    several times smaller than plain FP8's; without outliers the two are
    comparable."""
    B, H, N, d = 1, 2, 256, 128
    ratios = {}
    for outl in (0, 4):
        c = S.make_case(B, H, N, d, causal=True, seed=31, outliers=outl,
                        outlier_scale=16.0, scale=1.0 / (4 * np.sqrt(d)))
        o_ref, _ = ORA.attention_fwd(c["q"], c["k"], c["v"], c["scale"], True)
        errs = []
        for signs in (None, S.rotation_signs(33, d)):
            r = m.fp8_forward(c["q"], c["k"], c["v"], c["scale"], True, signs)
            errs.append(np.sqrt(np.mean((r["o"] - o_ref) ** 2)))
        ratios[outl] = errs[0] / errs[1]
    assert ratios[4] > 2.0, ratios
    assert 0.5 < ratios[0] < 2.0, ratios


PINS = [pin_e4m3_table, pin_e4m3_torch, pin_e4m3_roundtrip, pin_fwht_scipy,
        pin_rotation_one_hot, pin_mx_exponent_bruteforce,
        pin_mx_quantize_bound, pin_fp8_exact_reduction, pin_fp8_layout,
        pin_fp8_outlier_claim]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_fp8_model_pin(pin):
    pin(F8)


# ------------------------------------------------- planted mistakes ----

MUTANTS = [
    ("ties_away", "n = np.rint(a / step)", "n = np.floor(a / step + 0.5)"),
    ("no_subnormals", "step = np.where(a < 2.0 ** -6, 2.0 ** -9,",
     "step = np.where(a < 2.0 ** -6, 2.0 ** -6,"),
    ("butterfly_sign", "np.stack([a + b, a - b], axis=-2)",
     "np.stack([a + b, b - a], axis=-2)"),
    ("signs_after_transform",
     "return fwht_f32(np.asarray(x, dtype=np.float32) * s)",
     "return fwht_f32(np.asarray(x, dtype=np.float32)) * s"),
    ("exponent_strict", "e = np.where(2.0 * f <= 1.75,", "e = np.where(2.0 * f < 1.75,"),
    ("exponent_one_low", "ex - 1 - 8, ex - 1 - 7)", "ex - 1 - 9, ex - 1 - 8)"),
    ("no_inverse_d", "sc = sc / d", "sc = sc"),
    ("only_q_rotated", "k = rotate_f32(k, signs)", "k = k"),
    ("block_of_16", "MX_BLOCK = 32", "MX_BLOCK = 16"),
]


def _mutant(old, new):
    with open(F8.__file__) as f:
        src = f.read()
    assert src.count(old) >= 1, old
    mod = types.ModuleType("oracle_fp8_mutant")
    exec(compile(src.replace(old, new), "oracle_fp8_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[x[0] for x in MUTANTS])
def test_planted_mistake_is_caught(name, old, new):
    mod = _mutant(old, new)
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except Exception:
            return
    pytest.fail(f"no pin caught the planted mistake {name}")
