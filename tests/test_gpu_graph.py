"""The attention forward and backward captured in a HIP graph and replayed.

Every entry point enqueues its kernels on the stream it is given and makes no
allocation, host synchronisation or memset there, so a caller can record a
training step's attention calls into a graph once and replay it.  Each test
records the calls on torch's capture stream, then replays the graph several
times: before each replay new values are copied into the captured input
buffers, eager library calls on other buffers run between replays, and every
replay is compared bit for bit with an eager call on the same inputs (the
kernels use no atomics, so the results are deterministic).
"""
import numpy as np
import pytest

import synthetic as S
from gpu_util import DEV, to_dev

pytestmark = pytest.mark.gpu


def _inputs(B, H, N, d, causal, seed):
    inp = S.make_case(B, H, N, d, "bf16", causal, seed=seed, backward=True)
    return [to_dev(inp, n) for n in ("q", "k", "v", "do")], inp["scale"]


def _eager_step(fa, q, k, v, do, scale, causal, kv_len=None):
    import torch
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    fa.fa_fwd_kvlen(q, k, v, kv_len, o, lse, scale, causal)
    g = [torch.empty_like(q) for _ in range(3)]
    if kv_len is None:
        fa.fa_bwd_noalloc(q, k, v, o, do, lse, *g, scale, causal)
    else:
        B, H, N, d = q.shape
        ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d),
                         dtype=torch.uint8, device=q.device)
        fa.fa_bwd_kvlen(q, k, v, o, do, lse, kv_len, *g, ws, scale, causal)
    return [o, lse, *g]


def _check_replays(shape, causal, seed, kv=None, replays=3):
    import torch
    import io_aware_tiled_amd as fa
    B, H, N, d = shape
    (q, k, v, do), scale = _inputs(B, H, N, d, causal, seed)
    kv_len = (None if kv is None else
              torch.tensor(kv, dtype=torch.int32, device=DEV))
    # Captured buffers: inputs, outputs and (for the key-padded backward) the
    # workspace, all allocated before capture.
    cq, ck, cv, cdo = (t.clone() for t in (q, k, v, do))
    co = torch.empty_like(q)
    clse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    cg = [torch.empty_like(q) for _ in range(3)]
    ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8,
                     device=DEV)

    def record():
        fa.fa_fwd_kvlen(cq, ck, cv, kv_len, co, clse, scale, causal)
        if kv_len is None:
            fa.fa_bwd_noalloc(cq, ck, cv, co, cdo, clse, *cg, scale, causal)
        else:
            fa.fa_bwd_kvlen(cq, ck, cv, co, cdo, clse, kv_len, *cg, ws, scale,
                            causal)

    # One eager run on the side stream first (library set-up: device
    # attributes and the scratch address are looked up outside capture).
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        record()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        record()
    torch.cuda.synchronize()

    names = ("O", "LSE", "dQ", "dK", "dV")
    for r in range(replays):
        (nq, nk, nv, ndo), _ = _inputs(B, H, N, d, causal, seed + 100 * (r + 1))
        for dst, src in zip((cq, ck, cv, cdo), (nq, nk, nv, ndo)):
            dst.copy_(src)
        graph.replay()
        # eager library work on other buffers between the replay and the
        # reference, as a training step's other layers would do
        other = _eager_step(fa, q, k, v, do, scale, causal, kv_len)
        torch.cuda.synchronize()
        ref = _eager_step(fa, nq, nk, nv, ndo, scale, causal, kv_len)
        torch.cuda.synchronize()
        got = [co, clse, *cg]
        for nm, a, b in zip(names, got, ref):
            same = torch.equal(a, b)
            print(f"[graph] {shape} causal={causal} kv={kv is not None} "
                  f"replay {r}: {nm} bitwise {same}", flush=True)
            assert same, (shape, r, nm)
        del other


def test_graph_replay_fwd_bwd_noalloc_d128():
    _check_replays((2, 4, 1000, 128), True, 811)


def test_graph_replay_fwd_bwd_noalloc_d64_noncausal():
    _check_replays((1, 6, 777, 64), False, 821)


def test_graph_replay_fwd_bwd_kvlen_workspace():
    # key padding, with a batch that sees no key at all and one at N
    _check_replays((4, 2, 640, 128), True, 831, kv=[0, 257, 640, 64])
