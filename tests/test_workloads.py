"""The seeded workloads have the shapes and load structure they claim (CPU)."""
import json
import os
import sys

import numpy as np

from workloads import CONFIGS, ZIPF_ALPHA, generate, shrink

sys.path.insert(0, os.path.join(os.path.dirname(__file__), "golden"))
from fit_zipf_alpha import loads, zipf_slope  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_zipf_prefill_load_slope_is_minus_one():
    fit = json.load(open(os.path.join(GOLDEN, "zipf_alpha.json")))
    assert fit["alpha"] == ZIPF_ALPHA
    c = loads(CONFIGS["qwen_prefill"], ZIPF_ALPHA)
    assert abs(zipf_slope(c) + 1.0) < 0.01
    assert c.sum() == 8192 * 10 and c.min() > 0
    assert c.tolist() and c.max() == fit["max"] and c.min() == fit["min"]


def test_generation_is_seeded_and_shaped():
    cfg = shrink(CONFIGS["ling_decode"], T=8, D=64, E=4, k=2, I=32, I_shared=32)
    a, b = generate(cfg, seed=3), generate(cfg, seed=3)
    assert a.w13.shape == (4, 64, 64) and a.w2.shape == (4, 64, 32)
    assert a.s13.shape == (4, 64) and a.s2.shape == (4, 64)
    assert a.w13s.shape == (64, 64) and a.w2s.shape == (64, 32)
    for n in ("x", "wr", "w13", "w2", "s13", "s2", "w13s", "w2s"):
        ta, tb = getattr(a, n), getattr(b, n)
        assert ta.dtype == tb.dtype
        assert np.array_equal(ta.view(torch_u8(ta)).numpy(), tb.view(torch_u8(tb)).numpy())


def torch_u8(t):
    import torch
    return torch.uint8
