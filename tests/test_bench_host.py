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


def test_linear_backward_counts():
    """FLOPs and compulsory bytes of the linear-attention backward: 12d per
    visible pair inside a chunk and 10d^2 per row; Q, K, V, dO read and dQ,
    dK, dV written once."""
    w = S.WORKLOADS["linear_causal_fwd_bwd_d128"]
    assert w.backward and w.linear
    assert bench.linear_bwd_flops(w) == 64 * (12.0 * 128 * 64 * (64 * 65 // 2)
                                              + 10.0 * 4096 * 128 * 128)
    t = 4 * 16 * 4096 * 128 * 2
    assert bench.algorithmic_bytes(w, "linear_bwd") == 7 * t


def test_summarize_trace_keeps_timed_dispatches(tmp_path, monkeypatch):
    """The kernel-trace summary skips each kernel's warmup dispatches and
    keeps the next `steps` ones."""
    import csv
    path = tmp_path / "trace.csv"
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(["Kernel_Name", "Dispatch_Id", "Start_Timestamp",
                     "End_Timestamp"])
        for i in range(8):   # 3 warmup dispatches of 900 ns, 5 timed of 100
            wr.writerow(["void fa::k(int)", i, 0, 900 if i < 3 else 100])
        wr.writerow(["void other(int)", 99, 0, 5])
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    w = S.WORKLOADS["tiny_f32"]
    assert bench.summarize_trace(w, str(path), "cmd", 3, 5) == 0
    text = (tmp_path / "kernels_tiny_f32.md").read_text()
    assert "| `fa::k` | 5 | 0.1 | 0.1 | 0.1 |" in text


def test_summarize_trace_kernel_run_twice_per_step(tmp_path, monkeypatch):
    """A kernel the step runs twice: the dispatches of the warmup steps (2
    per step) are skipped and those of the timed steps (2 per step) kept."""
    import csv
    path = tmp_path / "trace.csv"
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(["Kernel_Name", "Dispatch_Id", "Start_Timestamp",
                     "End_Timestamp"])
        for i in range(16):  # 3 warmup steps x 2 of 900 ns, 5 timed x 2 of 100
            wr.writerow(["void fa::k(int)", i, 0, 900 if i < 6 else 100])
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    w = S.WORKLOADS["tiny_f32"]
    assert bench.summarize_trace(w, str(path), "cmd", 3, 5) == 0
    text = (tmp_path / "kernels_tiny_f32.md").read_text()
    assert "| `fa::k` | 10 | 0.1 | 0.1 | 0.1 |" in text


def test_summarize_trace_steady_pass(tmp_path, monkeypatch):
    """With a steady-state pass (7 untimed steps, then 5 timed ones after
    the 3 warmup and 5 timed steps), a kernel run twice per step keeps its
    timed dispatches and reports the last 5 steps beside them; a dispatch
    count that does not fit the run's steps is an error."""
    import csv
    path = tmp_path / "trace.csv"
    n = 2 * (3 + 5 + 7 + 5)
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(["Kernel_Name", "Dispatch_Id", "Start_Timestamp",
                     "End_Timestamp"])
        for i in range(n):   # warmup 900 ns, timed 100, untimed 700, last 300
            ns = 900 if i < 6 else 100 if i < 16 else 700 if i < 30 else 300
            wr.writerow(["void fa::k(int)", i, 0, ns])
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    w = S.WORKLOADS["tiny_f32"]
    assert bench.summarize_trace(w, str(path), "cmd", 3, 5, steady_warm=7) == 0
    text = (tmp_path / "kernels_tiny_f32.md").read_text()
    assert "| `fa::k` | 10 | 0.1 | 0.1 | 0.1 | 0.3 | 0.3 | 0.3 |" in text
    with pytest.raises(SystemExit):
        bench.summarize_trace(w, str(path), "cmd", 3, 5, steady_warm=6)


def test_summarize_stalls_fractions(tmp_path, monkeypatch):
    """The stall table gives wave-cycle counters as fractions of
    SQ_WAVE_CYCLES and instruction counts per MFMA."""
    import csv
    p1, p2 = tmp_path / "a.csv", tmp_path / "b.csv"
    rows1 = {"SQ_WAVE_CYCLES": 1000, "SQ_ACTIVE_INST_VALU": 250,
             "SQ_WAIT_INST_ANY": 400, "GRBM_GUI_ACTIVE": 8000}
    rows2 = {"SQ_INSTS_MFMA": 10, "SQ_INSTS_VALU": 35,
             "SQ_VALU_MFMA_BUSY_CYCLES": 512000, "GRBM_GUI_ACTIVE": 8000}
    for path, rows in ((p1, rows1), (p2, rows2)):
        with open(path, "w", newline="") as f:
            wr = csv.writer(f)
            wr.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
            for c, val in rows.items():
                wr.writerow(["void fa::bwd_dkdv_pipe_kernel<true>(int)", c, val])
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    w = S.WORKLOADS["tiny_f32"]
    assert bench.summarize_stalls(w, [str(p1), str(p2)], "cmd") == 0
    text = (tmp_path / "stalls_tiny_f32.md").read_text()
    line = [l for l in text.splitlines() if l.startswith("| bwd_dkdv")][0]
    cells = [c.strip() for c in line.strip("|").split("|")]
    assert cells[1] == "50.0%"          # 512000 / (1024 * 8000 / 8)
    assert cells[3] == "0.250"          # VALU / wave cycles
    assert cells[7] == "0.400"          # waiting to issue
    assert cells[10] == "3.50"          # VALU per MFMA


@pytest.mark.parametrize("causal,padded", [(True, False), (False, True)])
def test_standard_attention_matches_the_oracle(causal, padded):
    """The standard attention that the context comparison times computes
    attention (on the CPU here, float32): causal and key-padded cases
    against the fp64 oracle."""
    import torch
    rng = np.random.default_rng(7)
    B, H, N, d = 2, 2, 70, 16
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    kv = np.array([70, 33], dtype=np.int32) if padded else None
    scale = 1.0 / np.sqrt(d)
    t = lambda a: torch.from_numpy(a.astype(np.float32))
    o = bench.standard_attention(t(q), t(k), t(v), scale, causal,
                                 None if kv is None else torch.from_numpy(kv))
    ref, _ = oracle.attention_fwd(q, k, v, scale, causal=causal, kv_len=kv)
    assert np.abs(o.double().numpy() - ref).max() < 1e-5
