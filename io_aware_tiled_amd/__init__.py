"""Python binding of libfa: exact IO-aware tiled attention on MI355X (gfx950).

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of libfa.so (built in-tree by ``python -m io_aware_tiled_amd.build``);
PyTorch is used for device memory and for the current HIP stream.  There is
no CPU path and no fallback: if the library is missing or a tensor is not on
the GPU, the call raises.

The functions named like the C ABI (``fa_fwd``, ``fa_fwd_kvlen``,
``fa_fwd_block_sparse``, ``fa_fwd_f32``, ``fa_fp8_quantize``,
``fa_fwd_fp8_quantized``, ``fa_fwd_fp8``, ``fa_linear_fwd``, ``fa_bwd``,
``fa_bwd_preprocess``,
``fa_bwd_dkdv``, ``fa_bwd_dq``, the workspace-size queries,
``fa_status_string``, ``fa_version``) take caller-allocated tensors exactly
as the C calls take pointers.  ``forward``, ``forward_fp8``,
``linear_forward`` and ``backward``
allocate the outputs with ``torch.empty`` on the inputs' device and call
them.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "FAError", "lib", "lib_path", "fa_version", "fa_status_string",
    "fa_fwd", "fa_fwd_kvlen", "fa_fwd_f32", "fa_bwd_workspace_size",
    "fa_bwd", "fa_bwd_kvlen", "fa_bwd_noalloc", "BWD_NOALLOC_MAX_ROWS",
    "fa_bwd_preprocess", "fa_bwd_dkdv", "fa_bwd_dq",
    "fa_fwd_block_sparse", "fa_bwd_block_sparse", "fa_bwd_dkdv_block_sparse",
    "fa_bwd_dq_block_sparse", "fa_fp8_workspace_size",
    "fa_fp8_quantize",
    "fa_fwd_fp8_quantized", "fa_fwd_fp8", "fa_linear_fwd", "fa_linear_bwd",
    "linear_backward",
    "fa_linear_workspace_size", "fa_fwd_dropout", "fa_bwd_dropout",
    "fa_bwd_dkdv_dropout", "fa_bwd_dq_dropout", "dropout_threshold",
    "forward",
    "forward_fp8", "linear_forward", "backward", "EXPORTED_SYMBOLS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libfa.so")
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_S = ctypes.c_size_t
_U64 = ctypes.c_uint64
_U32 = ctypes.c_uint32

# name -> (restype, argtypes); mirrors include/fa.h
_SIGS = {
    "fa_version": (_I, []),
    "fa_status_string": (ctypes.c_char_p, [_I]),
    "fa_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P]),
    "fa_fwd_kvlen": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P]),
    "fa_fwd_block_sparse": (_I, [_P] * 6 + [_I, _I, _I, _I, _F, _I, _P]),
    "fa_fwd_f32": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P]),
    "fa_bwd_workspace_size": (_S, [_I, _I, _I, _I]),
    "fa_bwd": (_I, [_P] * 10 + [_S, _I, _I, _I, _I, _F, _I, _P]),
    "fa_bwd_kvlen": (_I, [_P] * 11 + [_S, _I, _I, _I, _I, _F, _I, _P]),
    "fa_bwd_noalloc": (_I, [_P] * 9 + [_I, _I, _I, _I, _F, _I, _P]),
    "fa_bwd_preprocess": (_I, [_P, _P, _P, _S, _I, _I, _I, _I, _P]),
    "fa_bwd_dkdv": (_I, [_P] * 8 + [_S, _I, _I, _I, _I, _F, _I, _P]),
    "fa_bwd_dq": (_I, [_P] * 7 + [_S, _I, _I, _I, _I, _F, _I, _P]),
    "fa_fp8_workspace_size": (_S, [_I, _I, _I, _I]),
    "fa_fp8_quantize": (_I, [_P] * 5 + [_S, _I, _I, _I, _I, _P]),
    "fa_fwd_fp8_quantized": (_I, [_P, _S, _P, _P, _I, _I, _I, _I, _F, _I, _P]),
    "fa_fwd_fp8": (_I, [_P] * 7 + [_S, _I, _I, _I, _I, _F, _I, _P]),
    "fa_linear_fwd": (_I, [_P] * 5 + [_S, _I, _I, _I, _I, _F, _P]),
    "fa_linear_workspace_size": (_S, [_I, _I, _I, _I]),
    "fa_linear_bwd": (_I, [_P] * 8 + [_S, _I, _I, _I, _I, _F, _P]),
    "fa_bwd_block_sparse": (_I, [_P] * 11 + [_S, _I, _I, _I, _I, _F, _I, _P]),
    "fa_bwd_dkdv_block_sparse": (_I, [_P] * 9 + [_S, _I, _I, _I, _I, _F, _I, _P]),
    "fa_bwd_dq_block_sparse": (_I, [_P] * 8 + [_S, _I, _I, _I, _I, _F, _I, _P]),
    "fa_fwd_dropout": (_I, [_P] * 5 + [_I, _I, _I, _I, _F, _I, _F, _U64, _U32, _P]),
    "fa_bwd_dropout": (_I, [_P] * 10 + [_S, _I, _I, _I, _I, _F, _I, _F, _U64,
                                        _U32, _P]),
    "fa_bwd_dkdv_dropout": (_I, [_P] * 8 + [_S, _I, _I, _I, _I, _F, _I, _F,
                                            _U64, _U32, _P]),
    "fa_bwd_dq_dropout": (_I, [_P] * 7 + [_S, _I, _I, _I, _I, _F, _I, _F, _U64,
                                          _U32, _P]),
}
EXPORTED_SYMBOLS = tuple(_SIGS)


class FAError(RuntimeError):
    """A libfa call returned a non-zero status."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fa_status_string(status)} (status {status})")


def lib_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Load libfa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with "
                "`python -m io_aware_tiled_amd.build` (no fallback exists)")
        handle = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def fa_version() -> int:
    return int(lib().fa_version())


def fa_status_string(status: int) -> str:
    return lib().fa_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise FAError(status, where)


# ---------------------------------------------------------------- marshalling

def _ptr(t):
    """Device pointer of a tensor (None -> NULL).  Refuses host tensors."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libfa takes GPU tensors only (no CPU path exists)")
    if not t.is_contiguous():
        raise ValueError("libfa takes contiguous tensors")
    return t.data_ptr()


def _stream(t, stream):
    import torch
    if stream is not None:
        return stream
    return torch.cuda.current_stream(t.device).cuda_stream


def _bhnd(q):
    if q.dim() != 4:
        raise ValueError(f"expected [B,H,N,d], got shape {tuple(q.shape)}")
    return tuple(int(x) for x in q.shape)


def _expect(t, dtype, shape, name):
    if t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {shape}, got {tuple(t.shape)}")


def fa_fwd(q, k, v, o, lse, scale, causal, stream=None):
    """C fa_fwd on bf16 tensors [B,H,N,d]; lse float32 [B,H,N]."""
    fa_fwd_kvlen(q, k, v, None, o, lse, scale, causal, stream)


def fa_fwd_kvlen(q, k, v, kv_len, o, lse, scale, causal, stream=None):
    """C fa_fwd_kvlen; kv_len is a device int32 [B] tensor or None."""
    import torch
    B, H, N, d = _bhnd(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _expect(t, torch.bfloat16, (B, H, N, d), n)
    _expect(lse, torch.float32, (B, H, N), "lse")
    if kv_len is not None:
        _expect(kv_len, torch.int32, (B,), "kv_len")
    st = lib().fa_fwd_kvlen(_ptr(q), _ptr(k), _ptr(v), _ptr(kv_len), _ptr(o),
                            _ptr(lse), B, H, N, d, float(scale), int(bool(causal)),
                            _stream(q, stream))
    _check(st, "fa_fwd_kvlen")


SPARSE_BQ, SPARSE_BK = 256, 128   # block-mask granularity (FA_SPARSE_BQ/BK)


def fa_fwd_block_sparse(q, k, v, block_mask, o, lse, scale, causal,
                        stream=None):
    """C fa_fwd_block_sparse; block_mask is a device uint8 tensor
    [H, ceil(N/256), ceil(N/128)] (nonzero = block kept)."""
    import torch
    B, H, N, d = _bhnd(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _expect(t, torch.bfloat16, (B, H, N, d), n)
    _expect(lse, torch.float32, (B, H, N), "lse")
    _expect(block_mask, torch.uint8,
            (H, -(-N // SPARSE_BQ), -(-N // SPARSE_BK)), "block_mask")
    st = lib().fa_fwd_block_sparse(_ptr(q), _ptr(k), _ptr(v),
                                   _ptr(block_mask), _ptr(o), _ptr(lse),
                                   B, H, N, d, float(scale),
                                   int(bool(causal)), _stream(q, stream))
    _check(st, "fa_fwd_block_sparse")


def fa_fwd_f32(q, k, v, o, lse, scale, causal, stream=None):
    """C fa_fwd_f32 on float32 tensors [B,H,N,d]."""
    import torch
    B, H, N, d = _bhnd(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _expect(t, torch.float32, (B, H, N, d), n)
    _expect(lse, torch.float32, (B, H, N), "lse")
    st = lib().fa_fwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                          B, H, N, d, float(scale), int(bool(causal)),
                          _stream(q, stream))
    _check(st, "fa_fwd_f32")


def fa_bwd_workspace_size(B, H, N, d) -> int:
    return int(lib().fa_bwd_workspace_size(int(B), int(H), int(N), int(d)))


def _ws(workspace):
    import torch
    if workspace.dtype != torch.uint8:
        raise ValueError("workspace must be a uint8 tensor")
    return _ptr(workspace), workspace.numel()


def fa_bwd(q, k, v, o, dO, lse, dq, dk, dv, workspace, scale, causal,
           stream=None):
    """C fa_bwd; workspace is a device uint8 tensor of at least
    fa_bwd_workspace_size bytes (torch allocations are 256-B aligned)."""
    import torch
    B, H, N, d = _bhnd(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dO, "dO"),
                 (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _expect(t, torch.bfloat16, (B, H, N, d), n)
    _expect(lse, torch.float32, (B, H, N), "lse")
    wp, wn = _ws(workspace)
    st = lib().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse),
                      _ptr(dq), _ptr(dk), _ptr(dv), wp, wn, B, H, N, d,
                      float(scale), int(bool(causal)), _stream(q, stream))
    _check(st, "fa_bwd")


def fa_bwd_noalloc(q, k, v, o, dO, lse, dq, dk, dv, scale, causal,
                   stream=None):
    """C fa_bwd_noalloc: fa_bwd with its D rows in the library's fixed
    per-device scratch instead of a workspace (B*H*N at most
    BWD_NOALLOC_MAX_ROWS); allocates nothing.  Calls that overlap on one GPU
    race on that scratch."""
    import torch
    B, H, N, d = _bhnd(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dO, "dO"),
                 (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _expect(t, torch.bfloat16, (B, H, N, d), n)
    _expect(lse, torch.float32, (B, H, N), "lse")
    st = lib().fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO),
                              _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), B, H, N,
                              d, float(scale), int(bool(causal)),
                              _stream(q, stream))
    _check(st, "fa_bwd_noalloc")


BWD_NOALLOC_MAX_ROWS = 1 << 21   # FA_BWD_NOALLOC_MAX_ROWS


def fa_bwd_kvlen(q, k, v, o, dO, lse, kv_len, dq, dk, dv, workspace, scale,
                 causal, stream=None):
    """C fa_bwd_kvlen: backward of fa_fwd_kvlen (kv_len: device int32 [B]
    or None)."""
    import torch
    B, H, N, d = _bhnd(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dO, "dO"),
                 (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _expect(t, torch.bfloat16, (B, H, N, d), n)
    _expect(lse, torch.float32, (B, H, N), "lse")
    kp = None
    if kv_len is not None:
        _expect(kv_len, torch.int32, (B,), "kv_len")
        kp = _ptr(kv_len)
    wp, wn = _ws(workspace)
    st = lib().fa_bwd_kvlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO),
                            _ptr(lse), kp, _ptr(dq), _ptr(dk), _ptr(dv), wp, wn,
                            B, H, N, d, float(scale), int(bool(causal)),
                            _stream(q, stream))
    _check(st, "fa_bwd_kvlen")


def fa_bwd_block_sparse(q, k, v, o, dO, lse, block_mask, dq, dk, dv,
                        workspace, scale, causal, stream=None):
    """C fa_bwd_block_sparse: backward of fa_fwd_block_sparse with the same
    uint8 block mask [H, ceil(N/256), ceil(N/128)]."""
    import torch
    B, H, N, d = _bhnd(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dO, "dO"),
                 (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _expect(t, torch.bfloat16, (B, H, N, d), n)
    _expect(lse, torch.float32, (B, H, N), "lse")
    _expect(block_mask, torch.uint8,
            (H, -(-N // SPARSE_BQ), -(-N // SPARSE_BK)), "block_mask")
    wp, wn = _ws(workspace)
    st = lib().fa_bwd_block_sparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                   _ptr(dO), _ptr(lse), _ptr(block_mask),
                                   _ptr(dq), _ptr(dk), _ptr(dv), wp, wn, B, H,
                                   N, d, float(scale), int(bool(causal)),
                                   _stream(q, stream))
    _check(st, "fa_bwd_block_sparse")


def _expect_all(pairs, dtype, shape):
    for t, n in pairs:
        _expect(t, dtype, shape, n)


def _expect_stage(q, k, v, dO, lse, outs):
    """dtype and shape checks of the stage-level backward entry points: the
    C ABI sees only pointers and cannot check buffer sizes."""
    import torch
    B, H, N, d = _bhnd(q)
    _expect_all(((q, "q"), (k, "k"), (v, "v"), (dO, "dO")) + tuple(outs),
                torch.bfloat16, (B, H, N, d))
    _expect(lse, torch.float32, (B, H, N), "lse")
    return B, H, N, d


def _expect_mask(block_mask, H, N):
    import torch
    _expect(block_mask, torch.uint8,
            (H, -(-N // SPARSE_BQ), -(-N // SPARSE_BK)), "block_mask")


def fa_bwd_dkdv_block_sparse(q, k, v, dO, lse, block_mask, dk, dv,
                             workspace, scale, causal, stream=None):
    B, H, N, d = _expect_stage(q, k, v, dO, lse, ((dk, "dk"), (dv, "dv")))
    _expect_mask(block_mask, H, N)
    wp, wn = _ws(workspace)
    st = lib().fa_bwd_dkdv_block_sparse(
        _ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(lse), _ptr(block_mask),
        _ptr(dk), _ptr(dv), wp, wn, B, H, N, d, float(scale),
        int(bool(causal)), _stream(q, stream))
    _check(st, "fa_bwd_dkdv_block_sparse")


def fa_bwd_dq_block_sparse(q, k, v, dO, lse, block_mask, dq, workspace,
                           scale, causal, stream=None):
    B, H, N, d = _expect_stage(q, k, v, dO, lse, ((dq, "dq"),))
    _expect_mask(block_mask, H, N)
    wp, wn = _ws(workspace)
    st = lib().fa_bwd_dq_block_sparse(
        _ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(lse), _ptr(block_mask),
        _ptr(dq), wp, wn, B, H, N, d, float(scale), int(bool(causal)),
        _stream(q, stream))
    _check(st, "fa_bwd_dq_block_sparse")


def fa_bwd_preprocess(o, dO, workspace, stream=None):
    import torch
    B, H, N, d = _bhnd(o)
    _expect_all(((o, "o"), (dO, "dO")), torch.bfloat16, (B, H, N, d))
    wp, wn = _ws(workspace)
    st = lib().fa_bwd_preprocess(_ptr(o), _ptr(dO), wp, wn, B, H, N, d,
                                 _stream(o, stream))
    _check(st, "fa_bwd_preprocess")


def fa_bwd_dkdv(q, k, v, dO, lse, dk, dv, workspace, scale, causal,
                stream=None):
    B, H, N, d = _expect_stage(q, k, v, dO, lse, ((dk, "dk"), (dv, "dv")))
    wp, wn = _ws(workspace)
    st = lib().fa_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(lse),
                           _ptr(dk), _ptr(dv), wp, wn, B, H, N, d,
                           float(scale), int(bool(causal)), _stream(q, stream))
    _check(st, "fa_bwd_dkdv")


def fa_bwd_dq(q, k, v, dO, lse, dq, workspace, scale, causal, stream=None):
    B, H, N, d = _expect_stage(q, k, v, dO, lse, ((dq, "dq"),))
    wp, wn = _ws(workspace)
    st = lib().fa_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(lse),
                         _ptr(dq), wp, wn, B, H, N, d, float(scale),
                         int(bool(causal)), _stream(q, stream))
    _check(st, "fa_bwd_dq")


FP8_V_ROW_BYTES = 80


# ------------------------------------------------------------- dropout

def dropout_threshold(p_drop: float) -> int:
    """The byte threshold p8 = round(256 p) the library applies (keep
    probability (256 - p8) / 256)."""
    x = 256.0 * float(ctypes.c_float(p_drop).value)
    p8 = int(math.floor(x))
    frac = x - p8
    if frac > 0.5 or (frac == 0.5 and p8 % 2 == 1):
        p8 += 1
    return p8


def _seed(seed):
    seed = int(seed)
    if not 0 <= seed < 1 << 64:
        raise ValueError("seed must fit in 64 unsigned bits")
    return seed


def fa_fwd_dropout(q, k, v, o, lse, scale, causal, p_drop, seed, offset=0,
                   stream=None):
    """C fa_fwd_dropout: attention with dropout on the weights (Philox
    mask of (seed, offset), see include/fa.h)."""
    import torch
    B, H, N, d = _bhnd(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _expect(t, torch.bfloat16, (B, H, N, d), n)
    _expect(lse, torch.float32, (B, H, N), "lse")
    st = lib().fa_fwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                              B, H, N, d, float(scale), int(bool(causal)),
                              float(p_drop), _seed(seed), int(offset),
                              _stream(q, stream))
    _check(st, "fa_fwd_dropout")


def fa_bwd_dropout(q, k, v, o, dO, lse, dq, dk, dv, workspace, scale, causal,
                   p_drop, seed, offset=0, stream=None):
    """C fa_bwd_dropout: gradients of fa_fwd_dropout for the same mask."""
    import torch
    B, H, N, d = _bhnd(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dO, "dO"),
                 (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _expect(t, torch.bfloat16, (B, H, N, d), n)
    _expect(lse, torch.float32, (B, H, N), "lse")
    wp, wn = _ws(workspace)
    st = lib().fa_bwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO),
                              _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), wp, wn,
                              B, H, N, d, float(scale), int(bool(causal)),
                              float(p_drop), _seed(seed), int(offset),
                              _stream(q, stream))
    _check(st, "fa_bwd_dropout")


def fa_bwd_dkdv_dropout(q, k, v, dO, lse, dk, dv, workspace, scale, causal,
                        p_drop, seed, offset=0, stream=None):
    B, H, N, d = _expect_stage(q, k, v, dO, lse, ((dk, "dk"), (dv, "dv")))
    wp, wn = _ws(workspace)
    st = lib().fa_bwd_dkdv_dropout(
        _ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(lse), _ptr(dk), _ptr(dv),
        wp, wn, B, H, N, d, float(scale), int(bool(causal)), float(p_drop),
        _seed(seed), int(offset), _stream(q, stream))
    _check(st, "fa_bwd_dkdv_dropout")


def fa_bwd_dq_dropout(q, k, v, dO, lse, dq, workspace, scale, causal, p_drop,
                      seed, offset=0, stream=None):
    B, H, N, d = _expect_stage(q, k, v, dO, lse, ((dq, "dq"),))
    wp, wn = _ws(workspace)
    st = lib().fa_bwd_dq_dropout(
        _ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(lse), _ptr(dq), wp, wn, B,
        H, N, d, float(scale), int(bool(causal)), float(p_drop), _seed(seed),
        int(offset), _stream(q, stream))
    _check(st, "fa_bwd_dq_dropout")


def fp8_row_bytes(d: int) -> int:
    """FA_FP8_ROW_BYTES(d): bytes of one quantised Q or K row."""
    return 144 if d == 128 else 80


def fa_fp8_workspace_size(B, H, N, d) -> int:
    return int(lib().fa_fp8_workspace_size(int(B), int(H), int(N), int(d)))


def _signs(signs, d):
    import torch
    if signs is None:
        return None
    _expect(signs, torch.int8, (d,), "signs")
    return _ptr(signs)


def fa_fp8_quantize(q, k, v, signs, workspace, stream=None):
    """C fa_fp8_quantize: bf16 q, k, v [B,H,N,d]; signs: device int8 [d] or
    None (no rotation); workspace: device uint8 tensor."""
    import torch
    B, H, N, d = _bhnd(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _expect(t, torch.bfloat16, (B, H, N, d), n)
    wp, wn = _ws(workspace)
    st = lib().fa_fp8_quantize(_ptr(q), _ptr(k), _ptr(v), _signs(signs, d),
                               wp, wn, B, H, N, d, _stream(q, stream))
    _check(st, "fa_fp8_quantize")


def fa_fwd_fp8_quantized(workspace, o, lse, score_scale, causal,
                         stream=None):
    """C fa_fwd_fp8_quantized: attention on a quantised workspace; o bf16
    [B,H,N,d] gives the shape."""
    import torch
    B, H, N, d = _bhnd(o)
    _expect(o, torch.bfloat16, (B, H, N, d), "o")
    _expect(lse, torch.float32, (B, H, N), "lse")
    wp, wn = _ws(workspace)
    st = lib().fa_fwd_fp8_quantized(wp, wn, _ptr(o), _ptr(lse), B, H, N, d,
                                    float(score_scale), int(bool(causal)),
                                    _stream(o, stream))
    _check(st, "fa_fwd_fp8_quantized")


def fa_fwd_fp8(q, k, v, signs, o, lse, workspace, scale, causal,
               stream=None):
    """C fa_fwd_fp8: quantise (rotating with signs unless None), then
    attend; the workspace keeps the quantised operands."""
    import torch
    B, H, N, d = _bhnd(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _expect(t, torch.bfloat16, (B, H, N, d), n)
    _expect(lse, torch.float32, (B, H, N), "lse")
    wp, wn = _ws(workspace)
    st = lib().fa_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _signs(signs, d),
                          _ptr(o), _ptr(lse), wp, wn, B, H, N, d,
                          float(scale), int(bool(causal)), _stream(q, stream))
    _check(st, "fa_fwd_fp8")


def fa_linear_workspace_size(B, H, N, d) -> int:
    return int(lib().fa_linear_workspace_size(int(B), int(H), int(N), int(d)))


def fa_linear_fwd(q, k, v, o, scale, workspace=None, stream=None):
    """C fa_linear_fwd: causal linear attention on bf16 [B,H,N,d];
    workspace: device uint8 tensor of fa_linear_workspace_size bytes, or
    None when that size is 0."""
    import torch
    B, H, N, d = _bhnd(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _expect(t, torch.bfloat16, (B, H, N, d), n)
    wp, wn = (None, 0) if workspace is None else _ws(workspace)
    st = lib().fa_linear_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), wp, wn, B, H,
                             N, d, float(scale), _stream(q, stream))
    _check(st, "fa_linear_fwd")


def fa_linear_bwd(q, k, v, dO, dq, dk, dv, scale, workspace=None,
                  stream=None):
    """C fa_linear_bwd: gradients of causal linear attention (bf16
    [B,H,N,d]); workspace as fa_linear_fwd's."""
    import torch
    B, H, N, d = _bhnd(q)
    _expect_all(((q, "q"), (k, "k"), (v, "v"), (dO, "dO"), (dq, "dq"),
                 (dk, "dk"), (dv, "dv")), torch.bfloat16, (B, H, N, d))
    wp, wn = (None, 0) if workspace is None else _ws(workspace)
    st = lib().fa_linear_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(dq),
                             _ptr(dk), _ptr(dv), wp, wn, B, H, N, d,
                             float(scale), _stream(q, stream))
    _check(st, "fa_linear_bwd")


# ------------------------------------------------------------- convenience

def forward(q, k, v, *, causal=False, scale=None, kv_len=None,
            block_mask=None, stream=None):
    """Returns (o, lse).  bf16 inputs use fa_fwd_kvlen (fa_fwd_block_sparse
    with a block mask), float32 use fa_fwd_f32 (no padding, no mask)."""
    import torch
    B, H, N, d = _bhnd(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if q.dtype == torch.float32:
        if kv_len is not None or block_mask is not None:
            raise ValueError("fa_fwd_f32 has no key-padding or block-sparse "
                             "variant")
        fa_fwd_f32(q, k, v, o, lse, scale, causal, stream)
    elif block_mask is not None:
        if kv_len is not None:
            raise ValueError("fa_fwd_block_sparse has no key padding")
        fa_fwd_block_sparse(q, k, v, block_mask, o, lse, scale, causal,
                            stream)
    else:
        fa_fwd_kvlen(q, k, v, kv_len, o, lse, scale, causal, stream)
    return o, lse


def forward_fp8(q, k, v, signs=None, *, causal=False, scale=None,
                workspace=None, stream=None):
    """FP8 forward of bf16 q, k, v; returns (o, lse, workspace).  signs:
    device int8 [d] (rotation) or None (plain FP8)."""
    import torch
    B, H, N, d = _bhnd(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nbytes = fa_fp8_workspace_size(B, H, N, d)
    if nbytes == 0:
        raise FAError(-3 if d not in (64, 128) else -2, "fa_fp8_workspace_size")
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fa_fwd_fp8(q, k, v, signs, o, lse, workspace, scale, causal, stream)
    return o, lse, workspace


def linear_forward(q, k, v, *, scale=None, stream=None):
    """Causal linear attention O = scale tril(Q K^T) V (scale defaults to
    1/sqrt(d)); returns o."""
    import torch
    B, H, N, d = _bhnd(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    n = fa_linear_workspace_size(B, H, N, d)
    ws = torch.empty(n, dtype=torch.uint8, device=q.device) if n else None
    fa_linear_fwd(q, k, v, o, scale, ws, stream)
    return o


def linear_backward(q, k, v, dO, *, scale=None, stream=None):
    """Gradients (dq, dk, dv) of causal linear attention
    O = scale tril(Q K^T) V for the output gradient dO."""
    import torch
    B, H, N, d = _bhnd(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    n = fa_linear_workspace_size(B, H, N, d)
    ws = torch.empty(n, dtype=torch.uint8, device=q.device) if n else None
    fa_linear_bwd(q, k, v, dO, dq, dk, dv, scale, ws, stream)
    return dq, dk, dv


def backward(q, k, v, o, lse, dO, *, causal=False, scale=None, stream=None,
             workspace=None, block_mask=None, kv_len=None):
    """Returns (dq, dk, dv) for the bf16 forward (fa_bwd_block_sparse when a
    block mask is given, fa_bwd_kvlen with key lengths)."""
    import torch
    B, H, N, d = _bhnd(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nbytes = fa_bwd_workspace_size(B, H, N, d)
    if nbytes == 0:
        raise FAError(-3 if d not in (64, 128) else -2,
                      "fa_bwd_workspace_size")
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    if block_mask is not None:
        if kv_len is not None:
            raise ValueError("fa_bwd_block_sparse has no key padding")
        fa_bwd_block_sparse(q, k, v, o, dO, lse, block_mask, dq, dk, dv,
                            workspace, scale, causal, stream)
    elif kv_len is not None:
        fa_bwd_kvlen(q, k, v, o, dO, lse, kv_len, dq, dk, dv, workspace,
                     scale, causal, stream)
    else:
        fa_bwd(q, k, v, o, dO, lse, dq, dk, dv, workspace, scale, causal,
               stream)
    return dq, dk, dv
