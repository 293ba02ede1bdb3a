"""fa_bwd_noalloc (the backward with its D rows in the library's fixed
per-device scratch) against fa_bwd (the same kernels with a caller
workspace), through the C ABI.

Both entry points run the same three kernels and the backward has no atomics,
so their results must be bitwise equal; two calls in a row, the second on a
smaller problem, check that the scratch is reused correctly.
"""
import numpy as np
import pytest

import synthetic as S
from gpu_util import run_fwd, to_dev

pytestmark = pytest.mark.gpu


def _both(inp):
    import torch
    import io_aware_tiled_amd as fa
    o, lse = run_fwd(inp)
    q, k, v, do = (to_dev(inp, n) for n in ("q", "k", "v", "do"))
    B, H, N, d = q.shape
    ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8,
                     device=q.device)
    ref = [torch.empty_like(q) for _ in range(3)]
    fa.fa_bwd(q, k, v, o, do, lse, *ref, ws, inp["scale"], inp["causal"])
    got = [torch.full_like(q, float("nan")) for _ in range(3)]
    fa.fa_bwd_noalloc(q, k, v, o, do, lse, *got, inp["scale"], inp["causal"])
    torch.cuda.synchronize()
    return ref, got


def _same(name, ref, got):
    import torch
    for nm, r, g in zip(("dQ", "dK", "dV"), ref, got):
        diff = float((r.float() - g.float()).abs().max())
        print(f"[noalloc] {name} {nm}: max |diff| {diff:.3e}", flush=True)
        assert torch.equal(r, g), (name, nm, diff)


def test_noalloc_matches_fa_bwd_two_calls():
    big = S.make_case(2, 16, 700, 128, "bf16", True, seed=71, backward=True)
    _same("2x16x700x128 causal", *_both(big))
    small = S.make_case(1, 3, 300, 64, "bf16", False, seed=72, backward=True)
    _same("1x3x300x64 non-causal", *_both(small))


def test_noalloc_rejects_too_large_before_launch():
    import torch
    import io_aware_tiled_amd as fa
    n = fa.BWD_NOALLOC_MAX_ROWS + 64
    t = torch.zeros(1, 1, n, 64, dtype=torch.bfloat16, device="cuda:0")
    lse = torch.zeros(1, 1, n, dtype=torch.float32, device="cuda:0")
    with pytest.raises(fa.FAError) as e:
        fa.fa_bwd_noalloc(t, t, t, t, t, lse, t, t, t, 0.125, True)
    assert e.value.status == -8
