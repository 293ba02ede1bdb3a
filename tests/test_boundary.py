"""C-ABI boundary checks that need no GPU.

The library must load, export every function include/fa.h declares, and
reject bad arguments with the documented status codes before making any HIP
call (so these run on a machine without a GPU).
"""
import ctypes
import os
import re

import pytest

import io_aware_tiled_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

OK, NULL, SHAPE, HEADDIM, ALIGN, WORKSPACE, HIP, DROPOUT = 0, -1, -2, -3, -4, -5, -6, -7
TOO_LARGE = -8

pytestmark = pytest.mark.skipif(not os.path.exists(fa.lib_path()),
                                reason="libfa.so not built")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(fa_[a-z0-9_]+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_expected_calls():
    names = _declared_functions()
    for want in ["fa_fwd", "fa_fwd_kvlen", "fa_fwd_f32", "fa_bwd",
                 "fa_fwd_block_sparse", "fa_fp8_workspace_size",
                 "fa_fp8_quantize", "fa_fwd_fp8_quantized", "fa_fwd_fp8",
                 "fa_linear_fwd", "fa_linear_workspace_size",
                 "fa_bwd_block_sparse", "fa_bwd_dkdv_block_sparse",
                 "fa_bwd_dq_block_sparse", "fa_fwd_dropout",
                 "fa_bwd_dropout", "fa_bwd_dkdv_dropout", "fa_bwd_dq_dropout",
                 "fa_bwd_workspace_size", "fa_status_string", "fa_version",
                 "fa_bwd_preprocess", "fa_bwd_dkdv", "fa_bwd_dq"]:
        assert want in names


def test_library_exports_every_declared_symbol():
    raw = ctypes.CDLL(fa.lib_path())
    for name in _declared_functions():
        assert hasattr(raw, name), name
    assert set(_declared_functions()) == set(fa.EXPORTED_SYMBOLS)


def test_version_and_status_strings():
    assert fa.fa_version() == 10000
    seen = set()
    for code in (OK, NULL, SHAPE, HEADDIM, ALIGN, WORKSPACE, HIP, DROPOUT,
                 TOO_LARGE):
        s = fa.fa_status_string(code)
        assert s.startswith("FA_"), s
        seen.add(s)
    assert len(seen) == 9
    assert "unknown" in fa.fa_status_string(12345)


# Fake, never-dereferenced device addresses: validation fails before use.
A = 0x10000          # 16-byte aligned
MIS = 0x10002        # misaligned


def _fwd(q=A, k=A, v=A, o=A, lse=A, B=1, H=1, N=64, d=64, scale=0.125,
         causal=0, kv=None):
    return fa.lib().fa_fwd_kvlen(q, k, v, kv, o, lse, B, H, N, d, scale,
                                 causal, None)


def test_fwd_argument_errors():
    assert _fwd(q=None) == NULL
    assert _fwd(o=None) == NULL
    assert _fwd(lse=None) == NULL
    assert _fwd(B=0) == SHAPE
    assert _fwd(H=-1) == SHAPE
    assert _fwd(N=0) == SHAPE
    assert _fwd(B=1 << 16, H=1 << 16, N=1 << 16) == SHAPE
    assert _fwd(d=32) == HEADDIM
    assert _fwd(d=96) == HEADDIM
    assert _fwd(d=256) == HEADDIM
    assert _fwd(q=MIS) == ALIGN
    assert _fwd(lse=MIS) == ALIGN
    assert _fwd(kv=0x10001) == ALIGN
    L = fa.lib()
    assert L.fa_fwd(None, A, A, A, A, 1, 1, 64, 64, 0.1, 1, None) == NULL
    assert L.fa_fwd(A, A, A, A, A, 1, 1, 64, 48, 0.1, 1, None) == HEADDIM
    assert L.fa_fwd_f32(A, A, None, A, A, 1, 1, 64, 64, 0.1, 0, None) == NULL
    assert L.fa_fwd_f32(A, A, A, A, MIS, 1, 1, 64, 64, 0.1, 0, None) == ALIGN
    assert L.fa_fwd_f32(A, A, A, A, A, 1, 0, 64, 64, 0.1, 0, None) == SHAPE


def test_block_sparse_argument_errors():
    L = fa.lib()

    def sp(q=A, m=A, o=A, N=64, d=128, B=1):
        return L.fa_fwd_block_sparse(q, A, A, m, o, A, B, 2, N, d, 0.1, 1,
                                     None)
    assert sp(q=None) == NULL
    assert sp(m=None) == NULL
    assert sp(o=None) == NULL
    assert sp(B=0) == SHAPE
    assert sp(N=64 * 2048 + 1) == SHAPE       # more key blocks than the limit
    assert sp(d=96) == HEADDIM
    assert sp(o=MIS) == ALIGN


def test_block_sparse_bwd_argument_errors():
    L = fa.lib()
    nbytes = fa.fa_bwd_workspace_size(1, 2, 64, 128)
    W = 0x100000

    def sb(ptrs=None, N=64, d=128, ws=W, wsb=nbytes):
        p = ptrs or [A] * 10
        return L.fa_bwd_block_sparse(*p, ws, wsb, 1, 2, N, d, 0.1, 1, None)
    for i in range(10):
        p = [A] * 10
        p[i] = None
        assert sb(p) == NULL, i
    assert sb(d=96) == HEADDIM
    assert sb(N=64 * 2048 + 1, wsb=1 << 40) == SHAPE
    assert sb(ws=None) == WORKSPACE
    p = [A] * 10
    p[7] = MIS
    assert sb(p) == ALIGN
    assert L.fa_bwd_dkdv_block_sparse(A, A, A, A, A, None, A, A, W, nbytes,
                                      1, 2, 64, 128, 0.1, 1, None) == NULL
    assert L.fa_bwd_dq_block_sparse(A, A, A, A, A, A, A, W, 0, 1, 2, 64, 128,
                                    0.1, 1, None) == WORKSPACE
    assert L.fa_bwd_dq_block_sparse(A, A, A, A, A, A, A, W, nbytes, 1, 2, 64,
                                    96, 0.1, 1, None) == HEADDIM


def test_workspace_size():
    ws = fa.fa_bwd_workspace_size
    def a256(x):
        return (x + 255) // 256 * 256
    for B, H, N in [(1, 1, 1), (4, 16, 4096), (2, 3, 1000)]:
        assert ws(B, H, N, 128) == a256(B * H * N * 4)
    assert ws(1, 1, 64, 64) == a256(64 * 4)   # head dim 64 or 128
    assert ws(1, 1, 64, 96) == 0
    assert ws(0, 1, 64, 128) == 0
    assert ws(1, 1, -5, 128) == 0


def test_bwd_argument_errors():
    L = fa.lib()
    nbytes = fa.fa_bwd_workspace_size(1, 1, 64, 128)
    W = 0x100000                          # 256-byte aligned fake address

    def bwd(ptrs=None, ws=W, wsb=nbytes, d=128, N=64):
        p = ptrs or [A] * 9
        return L.fa_bwd(*p, ws, wsb, 1, 1, N, d, 0.088, 1, None)
    for i in range(9):
        p = [A] * 9
        p[i] = None
        assert bwd(p) == NULL, i
    assert bwd(d=96) == HEADDIM
    assert bwd(N=0) == SHAPE
    assert bwd(ws=None) == WORKSPACE
    assert bwd(ws=W + 16) == WORKSPACE    # not 256-byte aligned
    assert bwd(wsb=nbytes - 1) == WORKSPACE
    p = [A] * 9
    p[4] = MIS
    assert bwd(p) == ALIGN
    assert L.fa_bwd_preprocess(A, None, W, nbytes, 1, 1, 64, 128, None) == NULL
    assert L.fa_bwd_preprocess(A, A, W, 16, 1, 1, 64, 128, None) == WORKSPACE
    assert L.fa_bwd_dkdv(A, A, A, A, A, A, None, W, nbytes, 1, 1, 64, 128,
                         0.1, 1, None) == NULL
    assert L.fa_bwd_dq(A, A, A, A, A, None, W, nbytes, 1, 1, 64, 128, 0.1,
                       1, None) == NULL
    assert L.fa_bwd_dq(A, A, A, A, A, A, W, nbytes, 1, 1, 64, 32, 0.1,
                       1, None) == HEADDIM
    assert L.fa_bwd_dq(A, A, A, A, A, A, W, 0, 1, 1, 64, 128, 0.1,
                       1, None) == WORKSPACE


def test_fp8_workspace_size():
    ws = fa.fa_fp8_workspace_size
    for B, H, N, d in [(1, 1, 1, 64), (4, 16, 4096, 128), (2, 3, 1000, 128),
                       (1, 12, 23400, 64)]:
        Np = -(-N // 64) * 64
        rb = fa.fp8_row_bytes(d)
        assert ws(B, H, N, d) == 2 * B * H * Np * rb + B * H * (Np // 64) * d * 80
        assert ws(B, H, N, d) % 256 == 0
    assert ws(1, 1, 64, 96) == 0
    assert ws(0, 1, 64, 128) == 0


def test_fp8_argument_errors():
    L = fa.lib()
    nbytes = fa.fa_fp8_workspace_size(1, 2, 100, 128)
    W = 0x100000

    def quant(q=A, k=A, v=A, s=None, ws=W, wsb=nbytes, N=100, d=128):
        return L.fa_fp8_quantize(q, k, v, s, ws, wsb, 1, 2, N, d, None)

    def attn(ws=W, wsb=nbytes, o=A, lse=A, N=100, d=128):
        return L.fa_fwd_fp8_quantized(ws, wsb, o, lse, 1, 2, N, d, 0.01, 1,
                                      None)

    def full(q=A, o=A, ws=W, wsb=nbytes, d=128, N=100):
        return L.fa_fwd_fp8(q, A, A, A, o, A, ws, wsb, 1, 2, N, d, 0.08, 0,
                            None)
    assert quant(q=None) == NULL and quant(v=None) == NULL
    assert quant(N=0) == SHAPE and quant(d=32) == HEADDIM
    assert quant(k=MIS) == ALIGN
    assert quant(ws=None) == WORKSPACE and quant(ws=W + 64) == WORKSPACE
    assert quant(wsb=nbytes - 1) == WORKSPACE
    assert attn(o=None) == NULL and attn(lse=None) == NULL
    assert attn(d=256) == HEADDIM and attn(lse=MIS) == ALIGN
    assert attn(ws=None) == WORKSPACE and attn(wsb=16) == WORKSPACE
    assert full(q=None) == NULL and full(o=None) == NULL
    assert full(d=48) == HEADDIM and full(o=MIS) == ALIGN
    assert full(wsb=nbytes - 256) == WORKSPACE
    # The workspace of a larger N does not fit a smaller one's size.
    assert quant(N=200, wsb=nbytes) == WORKSPACE


def test_linear_argument_errors():
    L = fa.lib()

    W = 0x100000

    def lin(q=A, o=A, B=1, N=64, d=128, ws=None, wsb=0):
        return L.fa_linear_fwd(q, A, A, o, ws, wsb, B, 2, N, d, 0.1, None)
    assert lin(q=None) == NULL and lin(o=None) == NULL
    assert lin(B=0) == SHAPE and lin(N=-1) == SHAPE
    assert lin(d=32) == HEADDIM and lin(d=256) == HEADDIM
    assert lin(q=MIS) == ALIGN and lin(o=MIS) == ALIGN
    # a long sequence with few heads is split and needs the workspace
    n = fa.fa_linear_workspace_size(1, 2, 20000, 128)
    assert n > 0 and n % 256 == 0
    assert lin(N=20000) == WORKSPACE
    assert lin(N=20000, ws=W, wsb=n - 1) == WORKSPACE
    assert lin(N=20000, ws=W + 16, wsb=n) == WORKSPACE
    assert fa.fa_linear_workspace_size(4, 16, 4096, 128) == 0
    assert fa.fa_linear_workspace_size(1, 1, 64, 96) == 0

    def lb(ptrs=None, B=1, N=64, d=128, ws=None, wsb=0):
        p = ptrs or [A] * 7
        return L.fa_linear_bwd(*p, ws, wsb, B, 2, N, d, 0.1, None)
    for i in range(7):
        p = [A] * 7
        p[i] = None
        assert lb(p) == NULL, i
        p[i] = MIS
        assert lb(p) == ALIGN, i
    assert lb(B=0) == SHAPE and lb(d=96) == HEADDIM
    assert lb(N=20000) == WORKSPACE
    assert lb(N=20000, ws=W, wsb=n - 1) == WORKSPACE


def test_python_binding_refuses_host_tensors():
    import torch
    q = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.forward(q, q, q)


def test_dropout_argument_errors():
    """Drop probability outside [0, 255.5/256) (or NaN) is rejected before
    any launch, and so are the usual pointer, shape and workspace errors."""
    L = fa.lib()

    def fw(p=0.1, q=A, o=A, d=64, N=64):
        return L.fa_fwd_dropout(q, A, A, o, A, 1, 2, N, d, 0.1, 1, p, 7, 0,
                                None)
    assert fw(p=-0.01) == DROPOUT
    assert fw(p=1.0) == DROPOUT
    assert fw(p=255.5 / 256) == DROPOUT      # rounds to 256
    assert fw(p=float("nan")) == DROPOUT
    assert fw(q=None) == NULL
    assert fw(d=96) == HEADDIM
    assert fw(N=0) == SHAPE
    assert fw(o=MIS) == ALIGN
    nbytes = fa.fa_bwd_workspace_size(1, 2, 64, 128)
    W = 0x100000

    def bw(p=0.1, ptrs=None, d=128, ws=W, wsb=nbytes):
        pp = ptrs or [A] * 9
        return L.fa_bwd_dropout(*pp, ws, wsb, 1, 2, 64, d, 0.1, 1, p, 7, 0,
                                None)
    assert bw(p=1.5) == DROPOUT
    assert bw(p=-1.0) == DROPOUT
    for i in range(9):
        pp = [A] * 9
        pp[i] = None
        assert bw(ptrs=pp) == NULL, i
    assert bw(d=96) == HEADDIM
    assert bw(ws=None) == WORKSPACE
    assert bw(wsb=nbytes - 1) == WORKSPACE
    assert L.fa_bwd_dkdv_dropout(A, A, A, A, A, A, A, W, nbytes, 1, 2, 64, 128,
                                 0.1, 1, 2.0, 7, 0, None) == DROPOUT
    assert L.fa_bwd_dq_dropout(A, A, A, A, A, None, W, nbytes, 1, 2, 64, 128,
                               0.1, 1, 0.1, 7, 0, None) == NULL


def test_dropout_threshold_rounding():
    """p8 = round(256 p) in float32, ties to even; agrees with the oracle's."""
    import numpy as np
    import oracle.dropout as OD
    for p in (0.0, 0.1, 0.25, 0.5, 0.3, 1.5 / 256, 2.5 / 256, 0.99, 254.5 / 256):
        assert fa.dropout_threshold(p) == OD.threshold(p), p
    assert fa.dropout_threshold(1.5 / 256) == 2
    assert fa.dropout_threshold(2.5 / 256) == 2
    assert fa.dropout_threshold(0.5) == 128


def test_bwd_kvlen_argument_errors():
    L = fa.lib()
    nbytes = fa.fa_bwd_workspace_size(1, 2, 64, 128)
    W = 0x100000

    def bk(ptrs=None, kv=A, d=128, ws=W):
        p = ptrs or [A] * 9
        return L.fa_bwd_kvlen(p[0], p[1], p[2], p[3], p[4], p[5], kv, p[6],
                              p[7], p[8], ws, nbytes, 1, 2, 64, d, 0.1, 1, None)
    for i in range(9):
        p = [A] * 9
        p[i] = None
        assert bk(p) == NULL, i
    assert bk(d=96) == HEADDIM
    assert bk(kv=0x10002) == ALIGN
    assert bk(ws=None) == WORKSPACE


def test_stage_wrappers_check_dtype_and_shape():
    """The stage-level backward wrappers check every tensor's dtype and
    shape before marshalling (the C ABI sees only pointers and cannot check
    buffer sizes); the checks run before the host-tensor refusal, so they
    are testable without a GPU."""
    import torch
    B, H, N, d = 1, 2, 64, 128
    bf = lambda *s: torch.zeros(*s, dtype=torch.bfloat16)
    q, k, v, do, dq, dk, dv = (bf(B, H, N, d) for _ in range(7))
    lse = torch.zeros(B, H, N, dtype=torch.float32)
    ws = torch.zeros(16, dtype=torch.uint8)
    mask = torch.ones(H, 1, 1, dtype=torch.uint8)
    short = bf(B, H, N - 1, d)
    f32 = torch.zeros(B, H, N, d, dtype=torch.float32)
    calls = [
        lambda t: fa.fa_bwd_preprocess(t, do, ws),
        lambda t: fa.fa_bwd_dkdv(q, k, v, do, lse, t, dv, ws, 0.1, True),
        lambda t: fa.fa_bwd_dq(q, t, v, do, lse, dq, ws, 0.1, True),
        lambda t: fa.fa_bwd_dkdv_block_sparse(q, k, t, do, lse, mask, dk, dv,
                                              ws, 0.1, True),
        lambda t: fa.fa_bwd_dq_block_sparse(q, k, v, t, lse, mask, dq, ws,
                                            0.1, True),
        lambda t: fa.fa_bwd_dkdv_dropout(q, k, v, do, lse, dk, t, ws, 0.1,
                                         True, 0.1, 1),
        lambda t: fa.fa_bwd_dq_dropout(q, k, v, do, lse, t, ws, 0.1, True,
                                       0.1, 1),
    ]
    for call in calls:
        for bad in (short, f32):
            with pytest.raises(ValueError):
                call(bad)
    with pytest.raises(ValueError):    # LSE of the wrong length
        fa.fa_bwd_dq(q, k, v, do, lse[:, :, :-1], dq, ws, 0.1, True)
    with pytest.raises(ValueError):    # block mask of the wrong shape
        fa.fa_bwd_dq_block_sparse(q, k, v, do, lse, mask[:1], dq, ws, 0.1,
                                  True)


def test_bwd_noalloc_argument_errors():
    """fa_bwd_noalloc: argument errors, including a problem larger than the
    fixed scratch (B*H*N > FA_BWD_NOALLOC_MAX_ROWS), are returned before
    any HIP call."""
    L = fa.lib()
    max_rows = fa.BWD_NOALLOC_MAX_ROWS
    assert max_rows == 1 << 21

    def bwd(ptrs=None, B=1, H=1, N=64, d=128):
        p = ptrs or [A] * 9
        return L.fa_bwd_noalloc(*p, B, H, N, d, 0.088, 1, None)
    for i in range(9):
        p = [A] * 9
        p[i] = None
        assert bwd(p) == NULL, i
    assert bwd(d=96) == HEADDIM
    assert bwd(N=0) == SHAPE
    p = [A] * 9
    p[7] = MIS
    assert bwd(p) == ALIGN
    assert bwd(B=2, H=1, N=max_rows // 2 + 1) == TOO_LARGE
    assert bwd(B=16, H=16, N=max_rows // 256 + 1) == TOO_LARGE
    text = open(HEADER).read()
    assert "#define FA_BWD_NOALLOC_MAX_ROWS (1 << 21)" in text
