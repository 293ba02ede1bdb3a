"""Writes closed_forms.json and pages_figures.json in this folder.

Every expected value below is a closed form derived by hand from the attention
definition softmax(scale * Q K^T) V ("Is a full-day context better than a
10-minute context? Flash attention and the sequence-length question",
marketmaker.cc, section "Why attention is memory-bound") and its masking
("Causal masking"; masked_fill with -inf in "Integration").  This script only
evaluates those closed forms (ln 2, ln 3, ...); it calls neither the oracle nor
the HIP library.  Run from the repository root:
    python tests/golden/make_closed_forms.py
"""
import json
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
ln3 = math.log(3.0)

closed = {
    "_about": (
        "Hand-derived closed-form cases for softmax(scale*QK^T)V. Pages: 'Is a full-day "
        "context better than a 10-minute context? Flash attention and the sequence-length "
        "question' (marketmaker.cc), sections 'Why attention is memory-bound', 'Causal "
        "masking', 'Integration'; 'Flash-Attention 2 for performance optimisation' "
        "(Medium), section 'Attention' (rows of the distribution sum to one). Each case "
        "states its derivation; make_closed_forms.py evaluates the closed forms."),
    "cases": [
        {"name": "two_keys",
         "derivation": (
             "s = (ln 3, 0) so p = (3/4, 1/4); o = 3/4*(4,0) + 1/4*(0,8) = (3,2); "
             "lse = ln(3+1) = ln 4. Backward with dO = (1,0) per row: dP = (4,0), D = 3, "
             "dS = (3/4, -3/4); dQ = 3/4*k1 = (3/4 ln 3, 0); per row dK = (dS_j q) = "
             "((3/4,0),(-3/4,0)) and dV = (p_j dO) = ((3/4,0),(1/4,0)); the two identical "
             "query rows double dK and dV."),
         "scale": 1.0, "causal": False, "kv_len": None,
         "q": [[1.0, 0.0], [1.0, 0.0]], "k": [[ln3, 0.0], [0.0, 0.0]],
         "v": [[4.0, 0.0], [0.0, 8.0]], "do": [[1.0, 0.0], [1.0, 0.0]],
         "o": [[3.0, 2.0], [3.0, 2.0]], "lse": [math.log(4.0)] * 2,
         "dq": [[0.75 * ln3, 0.0]] * 2,
         "dk": [[1.5, 0.0], [-1.5, 0.0]],
         "dv": [[1.5, 0.0], [0.5, 0.0]]},
        {"name": "uniform_causal",
         "derivation": "Q = 0 makes every score 0, so row i averages V rows 0..i and lse_i = ln(i+1).",
         "scale": 0.5, "causal": True, "kv_len": None,
         "q": [[0.0, 0.0]] * 4, "k": [[1.0, 2.0], [-3.0, 0.5], [0.25, 0.0], [7.0, -1.0]],
         "v": [[1.0, 0.0], [0.0, 1.0], [2.0, 2.0], [4.0, -4.0]],
         "o": [[1.0, 0.0], [0.5, 0.5], [1.0, 1.0], [1.75, -0.25]],
         "lse": [0.0, math.log(2.0), ln3, math.log(4.0)]},
        {"name": "key_padding",
         "derivation": "kv_len = 2 hides key 2; Q = 0 so every row averages V rows 0 and 1; lse = ln 2.",
         "scale": 1.0, "causal": False, "kv_len": [2],
         "q": [[0.0, 0.0]] * 3, "k": [[1.0, 1.0], [2.0, -1.0], [100.0, 100.0]],
         "v": [[2.0, 4.0], [6.0, 0.0], [1000.0, 1000.0]],
         "o": [[4.0, 2.0]] * 3, "lse": [math.log(2.0)] * 3},
        {"name": "no_visible_key",
         "derivation": "kv_len = 0 leaves no visible key: O = 0 and lse = -inf (the stated reading).",
         "scale": 1.0, "causal": False, "kv_len": [0],
         "q": [[1.0, 2.0]] * 2, "k": [[1.0, 1.0], [2.0, -1.0]], "v": [[2.0, 4.0], [6.0, 0.0]],
         "o": [[0.0, 0.0]] * 2, "lse": ["-inf", "-inf"]},
        {"name": "single_key",
         "derivation": "N = 1: the only key has weight 1, O = V, lse = scale*q.k = 0.25*(2*3 - 1*4) = 0.5.",
         "scale": 0.25, "causal": True, "kv_len": None,
         "q": [[2.0, -1.0]], "k": [[3.0, 4.0]], "v": [[-5.0, 9.0]],
         "o": [[-5.0, 9.0]], "lse": [0.5]},
    ]}

pages = {
    "_about": (
        "Arithmetic the pages print. 'Is a full-day context better than a 10-minute "
        "context? ...' (marketmaker.cc), introduction: a trading day of 23,400 one-second "
        "steps with 12 float16 heads needs roughly 12.9 GB for the score matrix alone."),
    "N": 23400, "heads": 12, "bytes_per_score": 2, "pages_figure_GB": 12.9,
    "exact_bytes": 23400 * 23400 * 12 * 2,
    "reading": "The pages' 12.9 GB is approximate; the exact count is 13.14e9 bytes (12.24 GiB).",
}

with open(os.path.join(HERE, "closed_forms.json"), "w") as f:
    json.dump(closed, f, indent=1)
with open(os.path.join(HERE, "pages_figures.json"), "w") as f:
    json.dump(pages, f, indent=1)
