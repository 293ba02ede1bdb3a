"""GPU parity of the backward kernels against the fp64 oracle's analytic
gradients (max abs error <= 5e-2 for dQ, dK, dV), plus the gradient
invariants sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i at full size."""
import numpy as np
import pytest

import synthetic as S
from gpu_util import (TOL_GRAD, host64, max_err, rel_err, report, run_fwd,
                      to_dev)

pytestmark = pytest.mark.gpu


def _run_bwd(inp, o, lse):
    import torch
    import io_aware_tiled_amd as fa
    q, k, v, do = (to_dev(inp, n) for n in ("q", "k", "v", "do"))
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, causal=inp["causal"],
                             scale=inp["scale"])
    torch.cuda.synchronize()
    return dq, dk, dv


def _check_bwd(name, inp, heads=None):
    from oracle import attention_bwd
    o, lse = run_fwd(inp)
    dq, dk, dv = _run_bwd(inp, o, lse)
    sel = (lambda a: a) if heads is None else (lambda a: a[:, heads])
    ref = attention_bwd(sel(inp["q"]), sel(inp["k"]), sel(inp["v"]),
                        sel(inp["do"]), inp["scale"], inp["causal"],
                        workers=8)
    errs, rels = {}, {}
    for nm, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        errs[nm] = max_err(sel(host64(g)), r, f"{name} {nm}")
        rels[nm + "_rel"] = rel_err(errs[nm], r)
    report(name, **errs, **rels)
    for nm, e in errs.items():
        assert e <= TOL_GRAD, (name, nm, e)
    return dq, dk, dv


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 32, 64, 129, 300, 1000])
def test_bwd_ragged(causal, N):
    B, H = (1, 3) if N <= 300 else (1, 2)
    inp = S.make_case(B, H, N, 128, "bf16", causal, seed=100 + N + causal,
                      backward=True)
    _check_bwd(f"bwd causal={causal} N={N}", inp)


# Grids of at least 256 workgroups of 256 query rows select the pipelined dQ
# kernel, and grids of at least 256 128-key workgroups the pipelined dK/dV
# kernel (at head dim 64 too); many heads at small N reach them with a full
# oracle comparison.
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 65, 200])
def test_bwd_wide_grid(d, causal, N):
    inp = S.make_case(16, 16, N, d, "bf16", causal, seed=300 + N + causal + d,
                      backward=True)
    _check_bwd(f"wide bwd d={d} causal={causal} N={N}", inp)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("scale", [-0.08, 0.0])
def test_bwd_wide_grid_scales(d, scale):
    inp = S.make_case(16, 16, 100, d, "bf16", True, seed=17 + d, backward=True,
                      scale=scale)
    _check_bwd(f"wide bwd d={d} scale={scale}", inp)


def test_bwd_bitwise_repeatable():
    """No atomics anywhere in the backward: dQ, dK and dV are bit-identical
    across runs."""
    import torch
    inp = S.make_case(1, 4, 700, 128, "bf16", True, seed=5, backward=True)
    o, lse = run_fwd(inp)
    dq0, dk0, dv0 = _run_bwd(inp, o, lse)
    for _ in range(5):
        dq, dk, dv = _run_bwd(inp, o, lse)
        assert torch.equal(dk, dk0) and torch.equal(dv, dv0)
        assert torch.equal(dq, dq0)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 33, 64, 300, 1000])
def test_bwd_head_dim_64(causal, N):
    """Head dimension 64 on small grids (the 8-wavefront dK/dV and 4-wavefront
    dQ kernels)."""
    B, H = (1, 3) if N <= 300 else (2, 2)
    inp = S.make_case(B, H, N, 64, "bf16", causal, seed=500 + N + causal,
                      backward=True)
    _check_bwd(f"bwd d64 causal={causal} N={N}", inp)


def test_bwd_gpt2_shape_d64():
    """GPT-2-small-shaped training step (8 x 12 x 1024 x 64, causal): every
    head against the oracle and against the gradient invariants."""
    inp = S.make_case(8, 12, 1024, 64, "bf16", True, seed=31, backward=True)
    dq, dk, dv = _check_bwd("bwd gpt2 shape", inp)
    tol = 3 * TOL_GRAD * np.sqrt(1024)
    e1 = float(np.abs(dk.float().sum(dim=2).cpu().numpy()).max())
    e2 = float(np.abs(dv.float().sum(dim=2).cpu().numpy()
                      - inp["do"].astype(np.float64).sum(axis=2)).max())
    report("gpt2 invariants", sum_dK=e1, sum_dV_minus_sum_dO=e2)
    assert e1 <= tol and e2 <= tol


def test_bwd_rejects_unsupported_head_dims():
    """d = 96 has no kernel, dense, block-sparse or with dropout: rejected
    before any launch."""
    import torch
    import io_aware_tiled_amd as fa
    q = torch.zeros(1, 1, 64, 96, dtype=torch.bfloat16, device="cuda:0")
    lse = torch.zeros(1, 1, 64, dtype=torch.float32, device="cuda:0")
    with pytest.raises(fa.FAError):
        fa.backward(q, q, q, q, lse, q)
    m = torch.ones(1, 1, 1, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(fa.FAError):
        fa.backward(q, q, q, q, lse, q, block_mask=m)
    ws = torch.empty(fa.fa_bwd_workspace_size(1, 1, 64, 64), dtype=torch.uint8,
                     device="cuda:0")
    q96 = torch.zeros(1, 1, 64, 96, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(fa.FAError):
        fa.fa_bwd_dropout(q96, q96, q96, q96, q96, lse, q96, q96, q96, ws,
                          0.125, True, 0.1, 1)


def _check_bwd_kvlen(name, inp, heads=None):
    import torch
    import io_aware_tiled_amd as fa
    from gpu_util import kv_dev
    from oracle import attention_bwd
    o, lse = run_fwd(inp)
    q, k, v, do = (to_dev(inp, n) for n in ("q", "k", "v", "do"))
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, causal=inp["causal"],
                             scale=inp["scale"], kv_len=kv_dev(inp))
    torch.cuda.synchronize()
    sel = (lambda a: a) if heads is None else (lambda a: a[:, heads])
    ref = attention_bwd(sel(inp["q"]), sel(inp["k"]), sel(inp["v"]),
                        sel(inp["do"]), inp["scale"], inp["causal"],
                        inp["kv_len"], workers=8)
    errs = {nm: max_err(sel(host64(g)), r, f"{name} {nm}")
            for nm, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref)}
    report(name, **errs)
    for nm, e in errs.items():
        assert e <= TOL_GRAD, (name, nm, e)
    return dq, dk, dv


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_key_padding(d, causal):
    """Backward of the key-padded forward (fa_bwd_kvlen): per-batch key
    lengths 0, 5, a ragged value and N.  (With a single visible key, dV of
    that key is the sum of all 300 dO rows, |dV| ~ 20-40, whose bf16
    rounding alone exceeds the absolute bar; 5 keys keep |dV| small.)"""
    N = 300
    inp = S.make_case(4, 2, N, d, "bf16", causal, seed=40 + d + causal,
                      backward=True, kv_len=[0, 5, 217, N])
    dq, dk, dv = _check_bwd_kvlen(f"bwd kvlen d{d} causal={causal}", inp)
    assert float(dq[0].float().abs().max()) == 0.0      # no visible key
    assert float(dk[2, :, 217:].float().abs().max()) == 0.0
    assert float(dv[2, :, 217:].float().abs().max()) == 0.0


def test_bwd_key_padding_bert_shape():
    """BERT-large-shaped padded training step (16 x 16 x 512 x 64, lengths
    in [256, 512]): every head against the oracle."""
    inp = S.make_case(16, 16, 512, 64, "bf16", False, seed=41, backward=True,
                      kv_len=np.random.default_rng(309).integers(256, 513, 16))
    _check_bwd_kvlen("bwd kvlen bert shape", inp)


# Key lengths of the pipelined-grid case: none, tile and block edges (32,
# 64, 128, 256 and the full 300), one past and one before them, and ragged
# (no length below 8: a key seen by all 300 rows alone has |dV| ~ 20-40,
# whose bf16 rounding alone exceeds the absolute bar).
PIPE_KV = [0, 32, 128, 256, 300, 8, 63, 64, 65, 127, 129, 200, 255, 257, 299,
           17]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_key_padding_pipelined_grid(d, causal):
    """A grid that takes the pipelined dK/dV kernel (16 x 16 heads of 300
    rows; at head dim 64 the two-workgroups-per-CU form), every head
    against the oracle; a batch entry with no visible key gets dQ = 0, keys
    at or past kv_len get dK = dV = 0."""
    N = 300
    inp = S.make_case(16, 16, N, d, "bf16", causal, seed=42 + causal + d,
                      backward=True, kv_len=PIPE_KV)
    dq, dk, dv = _check_bwd_kvlen(f"bwd kvlen pipelined d={d} causal={causal}", inp)
    assert float(dq[0].float().abs().max()) == 0.0
    for b, L in enumerate(PIPE_KV):
        if L < N:
            assert float(dk[b, :, L:].float().abs().max()) == 0.0, (b, L)
            assert float(dv[b, :, L:].float().abs().max()) == 0.0, (b, L)
