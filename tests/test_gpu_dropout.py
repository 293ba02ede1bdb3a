"""GPU parity of attention with dropout (fa_fwd_dropout, fa_bwd_dropout)
against the fp64 oracle (oracle/dropout.py).

Page: "Is a full-day context better than a 10-minute context? Flash
attention and the sequence-length question" (marketmaker.cc blog),
"Integration" (the framework call's dropout probability).  Mask: Philox4x32-10
(Salmon, Moraes, Dror, Shaw, SC 2011), one byte per (query, key) pair.

The keep mask is integer work, so it is checked bit for bit: with V one-hot
on a window of keys, O[i, c] = P[i, w0 + c] Z[i, w0 + c] / keep, which is
zero exactly where the kernel dropped the pair.  O, LSE and the gradients are
then checked against the oracle with the bf16 tolerances (O <= 2e-2,
LSE <= 1e-3, gradients <= 5e-2) scaled by 1/keep where the keep probability
amplifies the kept weights' rounding (p > 0.5 only).
"""
import numpy as np
import pytest

import oracle.dropout as OD
import synthetic as S
from gpu_util import (DEV, TOL_BF16_LSE, TOL_BF16_O, TOL_GRAD, host64, max_err,
                      report, to_dev)

pytestmark = pytest.mark.gpu


def _p8(p):
    return OD.threshold(p)


def _fwd(inp, p, seed, offset, v=None):
    import torch
    import io_aware_tiled_amd as fa
    q, k = to_dev(inp, "q"), to_dev(inp, "k")
    v = to_dev(inp, "v") if v is None else v
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    fa.fa_fwd_dropout(q, k, v, o, lse, inp["scale"], inp["causal"], p, seed,
                      offset)
    torch.cuda.synchronize()
    return o, lse


def _gpu_mask(inp, p, seed, offset):
    """The kernel's keep mask, read through one-hot V windows: bool [B,H,N,N]
    (False also where the key is not visible)."""
    import torch
    B, H, N, d = inp["q"].shape
    z = np.zeros((B, H, N, N), dtype=bool)
    for w0 in range(0, N, d):
        n = min(d, N - w0)
        v = torch.zeros((B, H, N, d), dtype=torch.bfloat16, device=DEV)
        idx = torch.arange(n, device=DEV)
        v[:, :, w0 + idx, idx] = 1.0
        o, _ = _fwd(inp, p, seed, offset, v=v)
        z[:, :, :, w0:w0 + n] = (o[..., :n] != 0).cpu().numpy()
    return z


@pytest.mark.parametrize("B,H,N,d,causal,p", [
    (1, 2, 128, 128, False, 0.1), (2, 3, 300, 64, True, 0.5),
    (1, 2, 257, 128, True, 0.25), (1, 1, 1, 128, False, 0.5),
    (1, 2, 70, 64, False, 0.9)])
def test_dropout_mask_bitexact(B, H, N, d, causal, p):
    seed, offset = 0x0123456789ABCDEF + N, 3 + N
    inp = S.make_case(B, H, N, d, "bf16", causal, seed=700 + N + d)
    z = _gpu_mask(inp, p, seed, offset)
    p8 = _p8(p)
    bad = 0
    for b in range(B):
        for h in range(H):
            ref = OD.keep_mask(seed, offset, p8, b * H + h, np.arange(N), N)
            if causal:
                ref &= np.tri(N, dtype=bool)
            bad += int(np.count_nonzero(ref != z[b, h]))
    report(f"mask B{B} H{H} N{N} d{d} causal={causal} p={p}",
           mismatches=float(bad), kept=float(z.mean()))
    assert bad == 0


def _tols(p):
    kp = OD.keep_prob(_p8(p))
    amp = max(1.0, 0.5 / kp)       # kept weights are scaled by 1/keep
    return TOL_BF16_O * amp, TOL_GRAD * amp


@pytest.mark.parametrize("B,H,N,d,causal,p", [
    (1, 2, 300, 128, True, 0.1), (1, 2, 300, 128, False, 0.2),
    (2, 3, 129, 64, True, 0.5), (1, 2, 1000, 64, False, 0.3),
    (1, 1, 17, 128, True, 0.9)])
def test_dropout_fwd_parity(B, H, N, d, causal, p):
    seed, offset = 977 + N, 11
    inp = S.make_case(B, H, N, d, "bf16", causal, seed=710 + N + d)
    o, lse = _fwd(inp, p, seed, offset)
    ref_o, ref_l = OD.attention_dropout_fwd(inp["q"], inp["k"], inp["v"],
                                            inp["scale"], causal, _p8(p), seed,
                                            offset)
    eo = max_err(host64(o), ref_o, "O")
    el = max_err(host64(lse), ref_l, "LSE")
    tol_o, _ = _tols(p)
    report(f"dropout fwd B{B} H{H} N{N} d{d} causal={causal} p={p}", O=eo, LSE=el)
    assert eo <= tol_o and el <= TOL_BF16_LSE


def _bwd(inp, o, lse, p, seed, offset):
    import torch
    import io_aware_tiled_amd as fa
    q, k, v, do = (to_dev(inp, n) for n in ("q", "k", "v", "do"))
    B, H, N, d = q.shape
    ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8,
                     device=DEV)
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    fa.fa_bwd_dropout(q, k, v, o, do, lse, dq, dk, dv, ws, inp["scale"],
                      inp["causal"], p, seed, offset)
    torch.cuda.synchronize()
    return dq, dk, dv


@pytest.mark.parametrize("B,H,N,d,causal,p", [
    (1, 2, 300, 128, True, 0.1), (1, 2, 300, 128, False, 0.2),
    (2, 2, 129, 128, True, 0.5), (1, 3, 64, 128, False, 0.3),
    (1, 1, 1, 128, True, 0.5), (1, 2, 700, 128, True, 0.75),
    (1, 2, 300, 64, True, 0.1), (2, 3, 257, 64, False, 0.5),
    (1, 2, 1000, 64, True, 0.2)])
def test_dropout_bwd_parity(B, H, N, d, causal, p):
    seed, offset = 31337 + N, 5
    inp = S.make_case(B, H, N, d, "bf16", causal, seed=720 + N + d, backward=True)
    o, lse = _fwd(inp, p, seed, offset)
    dq, dk, dv = _bwd(inp, o, lse, p, seed, offset)
    ref = OD.attention_dropout_bwd(inp["q"], inp["k"], inp["v"], inp["do"],
                                   inp["scale"], causal, _p8(p), seed, offset)
    _, tol = _tols(p)
    errs = {nm: max_err(host64(g), r, nm)
            for nm, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref)}
    report(f"dropout bwd B{B} H{H} N{N} d{d} causal={causal} p={p}", **errs)
    for nm, e in errs.items():
        assert e <= tol, (nm, e, tol)


def test_dropout_zero_matches_dense_bitwise():
    """p = 0 keeps every pair: the dropout kernels give the dense kernels'
    bits (same arithmetic, same order) on a grid large enough that the dense
    calls take the same pipelined kernels."""
    import torch
    import io_aware_tiled_amd as fa
    inp = S.make_case(4, 16, 1040, 128, "bf16", True, seed=9, backward=True)
    q, k, v, do = (to_dev(inp, n) for n in ("q", "k", "v", "do"))
    o0, l0 = fa.forward(q, k, v, causal=True, scale=inp["scale"])
    o1, l1 = _fwd(inp, 0.0, 1, 0)
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    g0 = fa.backward(q, k, v, o0, l0, do, causal=True, scale=inp["scale"])
    g1 = _bwd(inp, o0, l0, 0.0, 1, 0)
    for a, b in zip(g0, g1):
        assert torch.equal(a, b)


def test_dropout_zero_matches_dense_bitwise_d64():
    """The same at head dim 64 (the 8-wavefront dK/dV and 4-wavefront dQ
    kernels take the dropout path)."""
    import torch
    import io_aware_tiled_amd as fa
    inp = S.make_case(2, 4, 600, 64, "bf16", True, seed=10, backward=True)
    q, k, v, do = (to_dev(inp, n) for n in ("q", "k", "v", "do"))
    o0, l0 = fa.forward(q, k, v, causal=True, scale=inp["scale"])
    g0 = fa.backward(q, k, v, o0, l0, do, causal=True, scale=inp["scale"])
    g1 = _bwd(inp, o0, l0, 0.0, 1, 0)
    for a, b in zip(g0, g1):
        assert torch.equal(a, b)


def test_dropout_repeatable_and_seeded():
    """Same (seed, offset): bit-identical outputs; another offset or seed:
    a different mask."""
    import torch
    inp = S.make_case(1, 4, 400, 128, "bf16", True, seed=12, backward=True)
    o0, l0 = _fwd(inp, 0.2, 99, 1)
    g0 = _bwd(inp, o0, l0, 0.2, 99, 1)
    for _ in range(3):
        o1, l1 = _fwd(inp, 0.2, 99, 1)
        assert torch.equal(o0, o1) and torch.equal(l0, l1)
        for a, b in zip(g0, _bwd(inp, o0, l0, 0.2, 99, 1)):
            assert torch.equal(a, b)
    o2, l2 = _fwd(inp, 0.2, 99, 2)
    o3, _ = _fwd(inp, 0.2, 98, 1)
    assert torch.equal(l0, l2)               # LSE does not depend on the mask
    assert not torch.equal(o0, o2) and not torch.equal(o0, o3)


def test_dropout_workload_sampled():
    """The benchmark's workload (4 x 16 x 4096 x 128, causal, p = 0.1) in the
    launch configuration it times: O and LSE of sampled rows of three heads
    and the full gradients of two heads against the oracle."""
    import torch
    inp = S.make_inputs("dropout_causal_fwd_bwd_d128")
    dr = inp["dropout"]
    p, seed, off = dr["p"], dr["seed"], dr["offset"]
    o, lse = _fwd(inp, p, seed, off)
    rows = np.unique(np.concatenate([np.arange(0, 40), np.arange(4060, 4096),
                                     np.random.default_rng(4).integers(0, 4096, 60)]))
    heads = [(0, 0), (1, 5), (3, 15)]
    eo = el = 0.0
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref_o, ref_l = OD.attention_dropout_fwd(
            inp["q"][sl], inp["k"][sl], inp["v"][sl], inp["scale"], True,
            _p8(p), seed, off, rows=rows, bh0=b * 16 + h)
        eo = max(eo, max_err(host64(o[b, h, rows]), ref_o[0, 0], "O"))
        el = max(el, max_err(host64(lse[b, h, rows]), ref_l[0, 0], "LSE"))
    report("dropout workload fwd sampled", O=eo, LSE=el)
    assert eo <= TOL_BF16_O and el <= TOL_BF16_LSE
    dq, dk, dv = _bwd(inp, o, lse, p, seed, off)
    for b, h in [(0, 3), (2, 9)]:
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = OD.attention_dropout_bwd(inp["q"][sl], inp["k"][sl], inp["v"][sl],
                                       inp["do"][sl], inp["scale"], True,
                                       _p8(p), seed, off, bh0=b * 16 + h)
        errs = {nm: max_err(host64(g[b:b + 1, h:h + 1]), r, nm)
                for nm, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref)}
        report(f"dropout workload bwd head ({b},{h})", **errs)
        for nm, e in errs.items():
            assert e <= TOL_GRAD, (nm, e)
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("scale", [-0.08, 0.0])
def test_dropout_scales(d, scale):
    """Negative and zero scales (the sign is folded into Q or K inside the
    kernels) with dropout, forward and backward."""
    seed, offset = 4242, 9
    inp = S.make_case(1, 2, 200, d, "bf16", True, seed=730 + d, backward=True,
                      scale=scale)
    o, lse = _fwd(inp, 0.25, seed, offset)
    p8 = _p8(0.25)
    ref_o, ref_l = OD.attention_dropout_fwd(inp["q"], inp["k"], inp["v"],
                                            inp["scale"], True, p8, seed, offset)
    eo = max_err(host64(o), ref_o, "O")
    el = max_err(host64(lse), ref_l, "LSE")
    dq, dk, dv = _bwd(inp, o, lse, 0.25, seed, offset)
    ref = OD.attention_dropout_bwd(inp["q"], inp["k"], inp["v"], inp["do"],
                                   inp["scale"], True, p8, seed, offset)
    errs = {nm: max_err(host64(g), r, nm)
            for nm, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref)}
    report(f"dropout scale={scale} d{d}", O=eo, LSE=el, **errs)
    assert eo <= TOL_BF16_O and el <= TOL_BF16_LSE
    for nm, e in errs.items():
        assert e <= TOL_GRAD, (nm, e)
