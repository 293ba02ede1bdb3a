"""Full-size workloads compared with the fp64 oracle element by element.

The trading-day forward (1 x 12 x 23400 x 64, causal, sinusoidal key drift)
and the head-dim-128 forward + backward (4 x 16 x 4096 x 128, causal) run
once on the GPU, in the launch configuration the benchmark times; every
element of O and LSE (and of dQ, dK, dV) is then compared with the oracle,
a few heads per test so that each test's oracle work stays within tens of
seconds on the host cores.  Tolerances (max abs error): O 2e-2, LSE 1e-3,
gradients 5e-2 ([MM] "Correctness check": the fused kernel's output is
compared with a plain fp64 evaluation on the same inputs).
"""
import os

import numpy as np
import pytest

import synthetic as S
from gpu_util import (TOL_BF16_LSE, TOL_BF16_O, TOL_GRAD, max_err,
                      rel_err, report, run_fwd, to_dev)

pytestmark = pytest.mark.gpu

WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))


@pytest.fixture(scope="module")
def tradingday():
    inp = S.make_inputs("tradingday_causal")
    o, lse = run_fwd(inp)
    return inp, o.float().cpu().numpy(), lse.cpu().numpy()


@pytest.fixture(scope="module")
def d128_step():
    import torch
    import io_aware_tiled_amd as fa
    inp = S.make_inputs("causal_fwd_bwd_d128")
    o, lse = run_fwd(inp)
    q, k, v, do = (to_dev(inp, n) for n in ("q", "k", "v", "do"))
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, causal=True,
                             scale=inp["scale"])
    torch.cuda.synchronize()
    out = {"o": o.float().cpu().numpy(), "lse": lse.cpu().numpy(),
           "dq": dq.float().cpu().numpy(), "dk": dk.float().cpu().numpy(),
           "dv": dv.float().cpu().numpy()}
    return inp, out


@pytest.mark.parametrize("h0", [0, 4, 8])
def test_tradingday_forward_all_rows(tradingday, h0):
    """Heads h0..h0+3 of the trading-day forward, all 23400 rows each."""
    from oracle import attention_fwd
    inp, o, lse = tradingday
    hs = slice(h0, h0 + 4)
    ro, rl = attention_fwd(inp["q"][:, hs], inp["k"][:, hs], inp["v"][:, hs],
                           inp["scale"], True, workers=WORKERS)
    eo = max_err(o[:, hs].astype(np.float64), ro, "tradingday O")
    el = max_err(lse[:, hs].astype(np.float64), rl, "tradingday LSE")
    report(f"tradingday_causal heads {h0}..{h0 + 3}", O=eo, LSE=el,
           O_rel=rel_err(eo, ro), LSE_rel=rel_err(el, rl))
    assert eo <= TOL_BF16_O and el <= TOL_BF16_LSE, (eo, el)


@pytest.mark.parametrize("b", [0, 1, 2, 3])
def test_d128_forward_backward_all_heads(d128_step, b):
    """Batch entry b (16 heads x 4096 rows) of the head-dim-128 training
    step: O, LSE, dQ, dK and dV, every element."""
    from oracle import attention_bwd, attention_fwd
    inp, out = d128_step
    sel = (lambda a: a[b:b + 1])
    ro, rl = attention_fwd(sel(inp["q"]), sel(inp["k"]), sel(inp["v"]),
                           inp["scale"], True, workers=WORKERS)
    errs = {"O": max_err(sel(out["o"]).astype(np.float64), ro, "O"),
            "LSE": max_err(sel(out["lse"]).astype(np.float64), rl, "LSE")}
    rg = attention_bwd(sel(inp["q"]), sel(inp["k"]), sel(inp["v"]),
                       sel(inp["do"]), inp["scale"], True, workers=WORKERS)
    for nm, r in zip(("dQ", "dK", "dV"), rg):
        errs[nm] = max_err(sel(out[nm.lower()]).astype(np.float64), r, nm)
    rels = {nm + "_rel": rel_err(errs[nm], r)
            for nm, r in zip(("O", "LSE", "dQ", "dK", "dV"), (ro, rl) + rg)}
    report(f"causal_fwd_bwd_d128 batch {b}", **errs, **rels)
    assert errs["O"] <= TOL_BF16_O and errs["LSE"] <= TOL_BF16_LSE, errs
    for nm in ("dQ", "dK", "dV"):
        assert errs[nm] <= TOL_GRAD, (nm, errs[nm])


def test_d128_gradient_invariants(d128_step):
    """Over every head: sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i (every
    row sees key 0).  Bound: per-key errors of at most 5e-2 (checked above
    element by element) that are independent rounding errors add up like
    sqrt(N); three times that."""
    inp, out = d128_step
    N = inp["q"].shape[2]
    tol = 3 * TOL_GRAD * np.sqrt(N)
    e1 = float(np.abs(out["dk"].astype(np.float64).sum(axis=2)).max())
    e2 = float(np.abs(out["dv"].astype(np.float64).sum(axis=2)
                      - inp["do"].astype(np.float64).sum(axis=2)).max())
    report("causal_fwd_bwd_d128 invariants", sum_dK=e1,
           sum_dV_minus_sum_dO=e2)
    assert e1 <= tol and e2 <= tol
