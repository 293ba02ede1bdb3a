"""Host-side logic of bench.py (no GPU): the CPU-baseline leg of every
workload runs on a shrunken copy of it, and the FLOP and byte counts agree
with direct formulas."""
import dataclasses

import numpy as np
import pytest

import bench
import oracle
import oracle.linear
import synthetic as S


@pytest.mark.parametrize("name", sorted(S.WORKLOADS))
def test_cpu_baseline_runs_for_every_workload(name):
    w = S.WORKLOADS[name]
    small = dataclasses.replace(w, B=1, H=2, N=min(w.N, 200))
    inp = S.make_inputs(small)
    r = bench.cpu_baseline(small, inp, target_s=0.05)
    assert r["kind"] == "oracle" and r["value"] > 0 and r["cores"] >= 1
    assert small.name in r["sample"]


def test_visible_pairs_and_flops():
    w = S.WORKLOADS["causal_fwd_bwd_d128"]
    assert bench.visible_pairs(w, None) == 4 * 16 * 4096 * 4097 // 2
    w = S.WORKLOADS["bert_keypad"]
    kv = S.make_inputs(dataclasses.replace(w, N=8))["kv_len"]
    assert bench.visible_pairs(dataclasses.replace(w, N=8), kv) == \
        16 * int(np.minimum(kv, 8).sum()) * 8
    w = S.WORKLOADS["linear_causal_d128"]
    assert bench.linear_flops(w) == 64 * (4.0 * 128 * 64 * (64 * 65 // 2)
                                          + 4.0 * 4096 * 128 * 128)
    assert oracle.linear.linear_pairs(64) == 64 * 65 // 2


def test_block_sparse_pairs_match_element_mask():
    w = dataclasses.replace(S.WORKLOADS["blocksparse_d128"], B=1, H=2, N=700)
    inp = S.make_inputs(w)
    bm = inp["block_mask"]
    want = sum(int(oracle.visible_mask(0, 700, 700, False, None,
                                       block_mask=bm[h].astype(bool)).sum())
               for h in range(2))
    assert bench.visible_pairs(w, None, bm) == want


def test_algorithmic_bytes():
    w = S.WORKLOADS["fp8_causal_d128"]
    t = 4 * 16 * 4096 * 128 * 2
    ws = 2 * 64 * 4096 * 144 + 64 * 64 * 128 * 80
    assert bench.fp8_workspace_bytes(w) == ws
    assert bench.algorithmic_bytes(w, "fp8_quantize") == 3 * t + ws
    assert bench.algorithmic_bytes(S.WORKLOADS["linear_causal_d128"],
                                   "linear_fwd") == 4 * t
