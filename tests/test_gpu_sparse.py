"""GPU parity of the block-sparse forward (fa_fwd_block_sparse) against the
fp64 oracle restricted by the same block mask.

Block mask: one byte per 256 query rows x 128 keys and head; the oracle
expands it to an element mask.  Tolerances as the dense bf16 forward:
max abs error O 2e-2, LSE 1e-3.
"""
import numpy as np
import pytest

import synthetic as S
from gpu_util import (DEV, TOL_BF16_LSE, TOL_BF16_O, host64, max_err,
                      rel_err, report, to_dev)

pytestmark = pytest.mark.gpu


def _run_sparse(inp, mask):
    import torch
    import io_aware_tiled_amd as fa
    q, k, v = (to_dev(inp, n) for n in ("q", "k", "v"))
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    m = torch.from_numpy(np.ascontiguousarray(mask, dtype=np.uint8)).to(DEV)
    fa.fa_fwd_block_sparse(q, k, v, m, o, lse, inp["scale"], inp["causal"])
    torch.cuda.synchronize()
    return o, lse


def _check(name, inp, mask, rows=None, heads=None):
    from oracle import attention_fwd
    o, lse = _run_sparse(inp, mask)
    q, k, v = inp["q"], inp["k"], inp["v"]
    bm = mask.astype(bool)
    if heads is not None:
        q, k, v, bm = q[:, heads], k[:, heads], v[:, heads], bm[heads]
    oo, lo = attention_fwd(q, k, v, inp["scale"], inp["causal"], rows=rows,
                           block_mask=bm, workers=8)
    og, lg = host64(o), host64(lse)
    if heads is not None:
        og, lg = og[:, heads], lg[:, heads]
    if rows is not None:
        og, lg = og[:, :, rows], lg[:, :, rows]
    eo = max_err(og, oo, name + " O")
    el = max_err(lg, lo, name + " LSE")
    report(name, O=eo, LSE=el, O_rel=rel_err(eo, oo), LSE_rel=rel_err(el, lo))
    assert eo <= TOL_BF16_O and el <= TOL_BF16_LSE, (name, eo, el)
    return o, lse


def _mask(seed, H, N, density, empty_row=True):
    m = S.block_mask(seed, H, N, density)
    if empty_row and m.shape[1] > 1:
        m[0, 1, :] = 0                  # a block row with no visible key
    return m


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 64, 300, 1000])
def test_sparse_small_grid(d, causal, N):
    inp = S.make_case(2, 3, N, d, "bf16", causal, seed=40 + N + d)
    _check(f"sparse d={d} causal={causal} N={N}", inp,
           _mask(N + d, 3, N, 0.4))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_sparse_wide_grid(d, causal):
    # 2 x 64 heads x 4 query blocks: the grids of the large-grid kernel
    # variants (head dim 64 with two 32-row blocks per wavefront).
    inp = S.make_case(2, 64, 1000, d, "bf16", causal, seed=7 + d)
    _check(f"sparse wide d={d} causal={causal}", inp,
           _mask(99 + d, 64, 1000, 0.5), heads=slice(0, 64, 9))


def test_sparse_density_extremes():
    for density in (0.05, 0.95):
        inp = S.make_case(1, 4, 777, 128, "bf16", False, seed=8)
        _check(f"sparse density={density}", inp,
               _mask(5, 4, 777, density, empty_row=False))


def test_sparse_all_ones_equals_dense_bitwise():
    """With every block kept, the block-sparse kernel walks every tile and
    must return the dense kernel's bits (same grid, same kernel shape)."""
    import torch
    from gpu_util import run_fwd
    for d in (64, 128):
        inp = S.make_case(2, 64, 600, d, "bf16", True, seed=12 + d)
        ones = np.ones((64, 3, 5), dtype=np.uint8)
        o, lse = _run_sparse(inp, ones)
        od, lsed = run_fwd(inp)
        assert torch.equal(o.view(torch.int16), od.view(torch.int16)), d
        assert torch.equal(lse, lsed), d


def test_sparse_empty_mask():
    import torch
    inp = S.make_case(1, 2, 200, 64, "bf16", True, seed=13)
    o, lse = _run_sparse(inp, np.zeros((2, 1, 2), dtype=np.uint8))
    assert torch.all(o.float() == 0)
    assert torch.all(lse == -float("inf"))


def test_sparse_workload_sampled_rows():
    """The full block-sparse workload (4 x 16 x 4096, d = 128, half the
    blocks) on sampled rows of three heads."""
    inp = S.make_inputs("blocksparse_d128")
    rng = np.random.default_rng(0)
    rows = np.sort(np.concatenate([rng.choice(4096, 40, replace=False),
                                   [0, 255, 256, 4095]]))
    _check("blocksparse_d128 sampled", inp, inp["block_mask"], rows=rows,
           heads=[0, 7, 15])


# ---------------------------------------------------------------- backward

def _check_bwd(name, inp, mask, heads=None):
    """fa_fwd_block_sparse then fa_bwd_block_sparse against the oracle's
    gradients under the same block mask (max abs error <= 5e-2)."""
    import torch
    import io_aware_tiled_amd as fa
    from oracle import attention_bwd
    from gpu_util import TOL_GRAD
    q, k, v, do = (to_dev(inp, n) for n in ("q", "k", "v", "do"))
    m = torch.from_numpy(np.ascontiguousarray(mask, dtype=np.uint8)).to(DEV)
    o, lse = fa.forward(q, k, v, causal=inp["causal"], scale=inp["scale"],
                        block_mask=m)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, causal=inp["causal"],
                             scale=inp["scale"], block_mask=m)
    torch.cuda.synchronize()
    sel = (lambda a: a) if heads is None else (lambda a: a[:, heads])
    bm = mask.astype(bool) if heads is None else mask.astype(bool)[heads]
    ref = attention_bwd(sel(inp["q"]), sel(inp["k"]), sel(inp["v"]),
                        sel(inp["do"]), inp["scale"], inp["causal"],
                        workers=8, block_mask=bm)
    errs = {}
    for nm, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        errs[nm] = max_err(sel(host64(g)), r, f"{name} {nm}")
    report(name, **errs)
    for nm, e in errs.items():
        assert e <= TOL_GRAD, (name, nm, e)
    return dq, dk, dv


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [64, 300, 1000])
def test_sparse_bwd_small(d, causal, N):
    inp = S.make_case(2, 3, N, d, "bf16", causal, seed=60 + N + d,
                      backward=True)
    _check_bwd(f"sparse bwd d{d} causal={causal} N={N}", inp,
               _mask(N + 7, 3, N, 0.4))


def test_sparse_bwd_d64_alternate_columns_and_empty_rows():
    """Head dim 64 (the pipelined kernels at head dim 64 with tile lists): a
    key column no query keeps gets dK = dV = 0, a block row with no kept
    block dQ = 0."""
    N, H = 640, 2
    tq, tk = -(-N // 256), -(-N // 128)
    m = np.zeros((H, tq, tk), dtype=np.uint8)
    m[0, :, 0::2] = 1
    m[1, :, 1::2] = 1
    m[1, 1, :] = 0
    inp = S.make_case(1, H, N, 64, "bf16", True, seed=64, backward=True)
    dq, dk, dv = _check_bwd("sparse bwd d64 columns/rows", inp, m)
    assert float(dk[0, 0, 128:256].float().abs().max()) == 0.0
    assert float(dv[0, 1, 0:128].float().abs().max()) == 0.0
    assert float(dq[0, 1, 256:512].float().abs().max()) == 0.0


def test_sparse_bwd_d64_all_ones_equals_dense_bitwise():
    """At head dim 64 on a grid that fills the chip (16 x 16 heads) both calls
    take the pipelined kernels, so an all-ones mask gives the dense result
    bit for bit."""
    import torch
    import io_aware_tiled_amd as fa
    inp = S.make_case(16, 16, 300, 64, "bf16", True, seed=65, backward=True)
    q, k, v, do = (to_dev(inp, n) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, causal=True, scale=inp["scale"])
    ones = torch.ones((16, 2, 3), dtype=torch.uint8, device=DEV)
    g_sparse = fa.backward(q, k, v, o, lse, do, causal=True,
                           scale=inp["scale"], block_mask=ones)
    g_dense = fa.backward(q, k, v, o, lse, do, causal=True, scale=inp["scale"])
    torch.cuda.synchronize()
    for a, b in zip(g_sparse, g_dense):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_sparse_bwd_alternate_columns():
    """Masks that keep every other 128-key column (every other dK/dV
    workgroup sees no query at all and must write dK = dV = 0)."""
    N, H = 640, 2
    tq, tk = -(-N // 256), -(-N // 128)
    m = np.zeros((H, tq, tk), dtype=np.uint8)
    m[0, :, 0::2] = 1          # even key columns only
    m[1, :, 1::2] = 1          # odd key columns only
    inp = S.make_case(1, H, N, 128, "bf16", False, seed=61, backward=True)
    dq, dk, dv = _check_bwd("sparse bwd alternate columns", inp, m)
    assert float(dk[0, 0, 128:256].float().abs().max()) == 0.0
    assert float(dv[0, 1, 0:128].float().abs().max()) == 0.0


def test_sparse_bwd_all_ones_equals_dense_bitwise():
    """With every block kept the block-sparse backward must return the
    dense backward's bits; the grid (4 x 64 heads, N = 300) makes the dense
    call take the same pipelined kernels that every block-sparse call
    takes."""
    import torch
    import io_aware_tiled_amd as fa
    inp = S.make_case(4, 64, 300, 128, "bf16", True, seed=62, backward=True)
    q, k, v, do = (to_dev(inp, n) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, causal=True, scale=inp["scale"])
    ones = torch.ones((64, 2, 3), dtype=torch.uint8, device=DEV)
    g_sparse = fa.backward(q, k, v, o, lse, do, causal=True,
                           scale=inp["scale"], block_mask=ones)
    g_dense = fa.backward(q, k, v, o, lse, do, causal=True, scale=inp["scale"])
    torch.cuda.synchronize()
    for a, b in zip(g_sparse, g_dense):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_sparse_bwd_empty_rows():
    """A block row with no kept block: its queries get dQ = 0 and add
    nothing to dK, dV."""
    inp = S.make_case(1, 3, 512, 128, "bf16", True, seed=63, backward=True)
    m = _mask(64, 3, 512, 0.5)           # row 1 of head 0 emptied
    dq, _, _ = _check_bwd("sparse bwd empty row", inp, m)
    assert float(dq[0, 0, 256:512].float().abs().max()) == 0.0


def test_sparse_bwd_workload_heads():
    """The block-sparse workload's shape (4 x 16 x 4096, half the blocks):
    two heads of batch 0 against the full oracle."""
    w = S.WORKLOADS["blocksparse_d128"]
    inp = S.make_case(1, w.H, w.N, w.d, "bf16", False, seed=64, backward=True)
    mask = S.block_mask(w.block_seed, w.H, w.N, w.block_density)
    _check_bwd("blocksparse_d128 shape bwd heads 0,11", inp, mask,
               heads=np.array([0, 11]))
