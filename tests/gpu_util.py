"""Helpers shared by the GPU parity tests: upload seeded inputs, call the HIP
library through its binding, compare with the fp64 oracle."""
from __future__ import annotations

import numpy as np

DEV = "cuda:0"

# Tolerances (max absolute error against the fp64 oracle).
TOL_BF16_O = 2e-2
TOL_BF16_LSE = 1e-3
TOL_F32 = 1e-5
TOL_GRAD = 5e-2


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def to_dev(inp: dict, name: str):
    """Upload inp[name + '_bits'] as bf16 or float32 on the GPU."""
    import torch
    bits = inp[name + "_bits"]
    if inp["dtype"] == "bf16":
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(
            DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.float32)).to(DEV)


def kv_dev(inp: dict):
    import torch
    if inp["kv_len"] is None:
        return None
    return torch.from_numpy(np.asarray(inp["kv_len"], dtype=np.int32)).to(DEV)


def host64(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def max_err(gpu: np.ndarray, ref: np.ndarray, what: str = "") -> float:
    """Max |gpu - ref| over all elements; non-finite entries (-inf LSE) must
    match exactly."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    fg, fr = np.isfinite(gpu), np.isfinite(ref)
    bad = np.argwhere(fg != fr)
    assert bad.size == 0, (what, "finite pattern differs at", bad[:5].tolist())
    assert np.array_equal(gpu[~fg], ref[~fr]), (what, "non-finite values differ")
    if not fr.any():
        return 0.0
    return float(np.max(np.abs(gpu[fr] - ref[fr])))


def run_fwd(inp: dict, o=None, lse=None):
    """Forward through the HIP library; returns device (o, lse)."""
    import torch
    import io_aware_tiled_amd as fa
    q, k, v = (to_dev(inp, n) for n in ("q", "k", "v"))
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    if inp["dtype"] == "f32":
        fa.fa_fwd_f32(q, k, v, o, lse, inp["scale"], inp["causal"])
    else:
        fa.fa_fwd_kvlen(q, k, v, kv_dev(inp), o, lse, inp["scale"],
                        inp["causal"])
    torch.cuda.synchronize()
    return o, lse


def oracle_fwd(inp: dict, rows=None, heads=None, workers=8):
    from oracle import attention_fwd
    q, k, v = inp["q"], inp["k"], inp["v"]
    kv = inp["kv_len"]
    if heads is not None:
        q, k, v = q[:, heads], k[:, heads], v[:, heads]
    return attention_fwd(q, k, v, inp["scale"], inp["causal"], kv, rows=rows,
                         workers=workers)


def rel_err(abs_err: float, ref: np.ndarray) -> float:
    """The pages' relative error, max|gpu - ref| / max|ref| (finite entries),
    reported beside the absolute error that the tests gate on."""
    r = np.asarray(ref, dtype=np.float64)
    r = np.abs(r[np.isfinite(r)])
    return abs_err / r.max() if r.size and r.max() > 0 else 0.0


def report(name: str, **errs) -> None:
    print(f"[parity] {name}: " + ", ".join(f"{k}={v:.3e}" for k, v in errs.items()),
          flush=True)
