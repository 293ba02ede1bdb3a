"""The seeded input generator: bf16 rounding and workload shapes (CPU)."""
import numpy as np
import torch

import synthetic as S


def test_bf16_rounding_matches_torch():
    x = np.concatenate([
        S.normal(7, (100000,)) * np.float32(30.0),
        np.array([1.0, -1.0, 0.0, -0.0, 1e-30, 3.0e38,
                  1.00390625, 1.01171875,            # exact ties (RNE)
                  np.float32(1.0) + np.float32(2 ** -9)], dtype=np.float32),
    ]).astype(np.float32)
    ours = S.bf16_round_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(ours.view(np.int16), theirs)
    back = S.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16)
                          .float().numpy())


def test_workload_shapes_and_seeds():
    w = S.WORKLOADS["gpt2_causal"]
    inp = S.make_inputs(w)
    assert inp["q"].shape == (8, 12, 1024, 64) and inp["q"].dtype == np.float32
    assert inp["q_bits"].dtype == np.uint16
    assert inp["causal"] and inp["kv_len"] is None
    assert inp["scale"] == 0.125
    # values are exactly bf16: low 16 bits are zero
    assert not (inp["k"].view(np.uint32) & 0xFFFF).any()
    # same seed -> same bits
    again = S.make_inputs(w)
    assert np.array_equal(again["v_bits"], inp["v_bits"])


def test_keypad_lengths_in_range():
    inp = S.make_inputs("bert_keypad", heads=slice(0, 1))
    kv = inp["kv_len"]
    assert kv.shape == (16,) and kv.dtype == np.int32
    assert kv.min() >= 256 and kv.max() <= 512
    assert inp["q"].shape == (16, 1, 512, 64)


def test_tradingday_drift():
    w = S.WORKLOADS["tradingday_causal"]
    assert w.N == 23400 and w.N % 390 == 0
    inp = S.make_inputs(w, heads=slice(0, 2))
    raw = S.normal(w.seeds[1], (w.B, w.H, w.N, w.d))[:, :2]
    t = np.arange(w.N)
    drift = (0.5 * np.sin(2 * np.pi * t / 390.0)).astype(np.float32)
    want = S.bf16_bits_to_f32(S.bf16_round_bits(raw + drift[None, None, :, None]))
    assert np.array_equal(inp["k"], want)
    # the drift is visible in the mean over channels and heads
    m = inp["k"][0].mean(axis=(0, 2))
    assert np.corrcoef(m, drift)[0, 1] > 0.9


def test_scale_is_float32_rounded():
    assert S.WORKLOADS["causal_fwd_bwd_d128"].scale == float(
        np.float32(1 / np.sqrt(128)))
