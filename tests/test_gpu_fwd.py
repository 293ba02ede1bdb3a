"""GPU parity of the forward kernels against the fp64 oracle.

Every case is compared element by element (every O entry and every LSE
entry, padded rows included).  The trading-day and head-dim-128 workloads,
whose oracle takes tens of seconds, are in test_gpu_full_configs.py.
Tolerances (max abs error): bf16 O 2e-2, LSE 1e-3; float32 O and LSE 1e-5.
"""
import numpy as np
import pytest

import synthetic as S
from gpu_util import (DEV, TOL_BF16_LSE, TOL_BF16_O, TOL_F32, host64,
                      max_err, oracle_fwd, rel_err, report, run_fwd)

pytestmark = pytest.mark.gpu


def _check(name, inp, rows=None, heads=None):
    o, lse = run_fwd(inp)
    oo, lo = oracle_fwd(inp, rows=rows, heads=heads)
    og, lg = host64(o), host64(lse)
    if heads is not None:
        og, lg = og[:, heads], lg[:, heads]
    if rows is not None:
        og, lg = og[:, :, rows], lg[:, :, rows]
    eo = max_err(og, oo, name + " O")
    el = max_err(lg, lo, name + " LSE")
    report(name, O=eo, LSE=el, O_rel=rel_err(eo, oo), LSE_rel=rel_err(el, lo))
    if inp["dtype"] == "f32":
        assert eo <= TOL_F32 and el <= TOL_F32, (name, eo, el)
    else:
        assert eo <= TOL_BF16_O and el <= TOL_BF16_LSE, (name, eo, el)
    return o, lse


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 63, 64, 65, 127, 129, 300, 1000])
def test_fwd_bf16_ragged(d, causal, N):
    B, H = (2, 3) if N <= 300 else (1, 2)
    inp = S.make_case(B, H, N, d, "bf16", causal, seed=N * 7 + d + causal)
    _check(f"bf16 d={d} causal={causal} N={N}", inp)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_kvlen_edges(d, causal):
    N = 300
    kv = [0, 1, 63, 64, 65, 129, 299, 300]
    inp = S.make_case(len(kv), 2, N, d, "bf16", causal, seed=11 + d, kv_len=kv)
    _check(f"kvlen d={d} causal={causal}", inp)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 33, 256, 300])
def test_fwd_f32(d, causal, N):
    inp = S.make_case(2, 2, N, d, "f32", causal, seed=5 + N + d)
    _check(f"f32 d={d} causal={causal} N={N}", inp)


def test_fwd_large_magnitude_scores():
    # Q scaled by 30: near one-hot rows, exp would overflow without the max.
    for d in (64, 128):
        inp = S.make_case(1, 2, 257, d, "bf16", True, seed=3, q_scale=30.0)
        _check(f"Q*30 d={d}", inp)


def test_fwd_negative_and_zero_scale():
    for scale in (-0.125, 0.0):
        inp = S.make_case(1, 2, 200, 64, "bf16", True, seed=4, scale=scale)
        _check(f"scale={scale}", inp)
        inp = S.make_case(1, 2, 100, 64, "f32", False, seed=4, scale=scale)
        _check(f"f32 scale={scale}", inp)


def test_fwd_padded_kv_contents_do_not_matter():
    """Keys at or past kv_len are masked: setting their K/V rows to huge
    finite values must leave O and LSE bit-identical."""
    import torch
    N, d = 300, 64
    kv = [7, 130, 300]
    inp = S.make_case(len(kv), 2, N, d, "bf16", False, seed=21, kv_len=kv)
    o1, l1 = run_fwd(inp)
    big = dict(inp)
    for name in ("k", "v"):
        bits = inp[name + "_bits"].copy()
        for b, L in enumerate(kv):
            bits[b, :, L:] = S.bf16_round_bits(np.full((1,), 3.0e4, np.float32))[0]
        big[name + "_bits"] = bits
    o2, l2 = run_fwd(big)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fwd_writes_nothing_outside_outputs():
    """Guard bands around O and LSE keep their sentinel values."""
    import torch
    B, H, N, d = 2, 3, 129, 64
    inp = S.make_case(B, H, N, d, "bf16", True, seed=31)
    G = 256
    n = B * H * N * d
    obuf = torch.full((n + 2 * G,), 7.0, dtype=torch.bfloat16, device=DEV)
    lbuf = torch.full((B * H * N + 2 * G,), 7.0, dtype=torch.float32, device=DEV)
    o = obuf[G:G + n].view(B, H, N, d)
    lse = lbuf[G:G + B * H * N].view(B, H, N)
    run_fwd(inp, o=o, lse=lse)
    assert bool((obuf[:G] == 7.0).all()) and bool((obuf[G + n:] == 7.0).all())
    assert bool((lbuf[:G] == 7.0).all()) and bool((lbuf[-G:] == 7.0).all())
    oo, lo = oracle_fwd(inp)
    assert max_err(host64(o), oo) <= TOL_BF16_O


def test_fwd_bitwise_repeatable():
    """No atomics in the forward: 20 runs give identical bits."""
    import torch
    inp = S.make_case(2, 4, 1000, 64, "bf16", True, seed=41)
    o0, l0 = run_fwd(inp)
    for _ in range(20):
        o, lse = run_fwd(inp)
        assert torch.equal(o, o0) and torch.equal(lse, l0)


# ------------------------------------------- wide grids (pipelined kernels)
# Grids of at least 256 blocks of 256 rows select the pipelined kernels
# (head dim 64: 128-row workgroups of one block per wavefront below 512
# such blocks, 256-row workgroups of two blocks per wavefront from 512;
# head dim 128: 256-row workgroups of 8 wavefronts).  Many heads at small
# N reach them with an oracle that still runs every row.

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,BH,N", [(64, (16, 16), 1), (64, (16, 16), 65),
                                    (64, (16, 16), 200), (64, (8, 32), 300),
                                    (64, (4, 64), 513), (128, (32, 16), 1),
                                    (128, (32, 16), 65), (128, (16, 32), 200),
                                    (128, (16, 16), 300)])
def test_fwd_wide_grid_ragged(causal, d, BH, N):
    B, H = BH
    inp = S.make_case(B, H, N, d, "bf16", causal, seed=N + d + 3 * causal)
    _check(f"wide d={d} B={B} H={H} N={N} causal={causal}", inp)


@pytest.mark.parametrize("d,B", [(64, 32), (64, 64), (128, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_wide_grid_kvlen(d, B, causal):
    N = 300
    rng = np.random.default_rng(77 + d + B)
    kv = rng.integers(0, N + 1, B)
    kv[:8] = [0, 1, 63, 64, 65, 256, 299, 300]
    inp = S.make_case(B, 4, N, d, "bf16", causal, seed=12 + d,
                      kv_len=kv.tolist())
    _check(f"wide kvlen d={d} B={B} causal={causal}", inp)


@pytest.mark.parametrize("d", [64, 128])
def test_fwd_wide_grid_large_magnitude_and_scale(d):
    H = 16 if d == 64 else 32
    inp = S.make_case(16, H, 257, d, "bf16", True, seed=9, q_scale=30.0)
    _check(f"wide Q*30 d={d}", inp)
    for scale in (-0.125, 0.0):
        inp = S.make_case(16, H, 200, d, "bf16", True, seed=4, scale=scale)
        _check(f"wide scale={scale} d={d}", inp)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_growing_scores(d, causal):
    """Scores that grow by ~100 (log2 units) along the keys: the reference
    max of a row must move many times, far past any fixed headroom."""
    H = 16 if d == 64 else 32
    N = 700
    inp = S.make_case(16, H, N, d, "bf16", causal, seed=61 + d)
    ramp = np.linspace(0.0, 60.0, N, dtype=np.float32)[None, None, :, None]
    kb = S.bf16_round_bits(inp["k"] + ramp)
    inp = dict(inp, k_bits=kb, k=S.bf16_bits_to_f32(kb))
    _check(f"growing scores d={d} causal={causal}", inp)


# ---------------------------------------------------------- full workloads

def test_workload_tiny_f32():
    _check("tiny_f32", S.make_inputs("tiny_f32"))


def test_workload_gpt2_causal():
    _check("gpt2_causal", S.make_inputs("gpt2_causal"))


def test_workload_bert_keypad():
    _check("bert_keypad", S.make_inputs("bert_keypad"))


# The trading-day and head-dim-128 workloads are compared in full (every O
# and LSE element) in test_gpu_full_configs.py.
