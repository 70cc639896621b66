"""Pins of the oracle's expert FFN, combine and whole layer (CPU only)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle.brute import brute_force_layer
from oracle.formats import decode
from oracle.moe import (expert_ffn, experts_from_bits, layer, layer_tokens,
                        permute, rel_err, shared_from_bits, topk_softmax)
from workloads import CONFIGS, generate, shrink, to_bits


def decoded(wl):
    c = wl.cfg
    x = decode(to_bits(wl.x), c.act_dtype)
    wr = decode(to_bits(wl.wr), c.act_dtype)
    s13 = None if wl.s13 is None else wl.s13.numpy()
    s2 = None if wl.s2 is None else wl.s2.numpy()
    experts = experts_from_bits(to_bits(wl.w13), s13, to_bits(wl.w2), s2, c.w_dtype)
    shared = None
    if c.I_shared:
        shared = shared_from_bits(to_bits(wl.w13s), None if wl.s13s is None else wl.s13s.numpy(),
                                  to_bits(wl.w2s), None if wl.s2s is None else wl.s2s.numpy(),
                                  c.shared_w_dtype)
    return x, wr, experts, shared


SMALL = {
    "tiny_fp32": CONFIGS["tiny_fp32"],
    "qwen_like": shrink(CONFIGS["qwen_decode"], T=24, D=128, E=32, k=10, I=64, I_shared=64),
    "qwen_zipf": shrink(CONFIGS["qwen_prefill"], T=40, D=128, E=32, k=10, I=64, I_shared=64),
    "gemma_like": shrink(CONFIGS["gemma"], T=32, D=128, E=16, k=8, I=64, I_shared=192),
    "ling_fp8": shrink(CONFIGS["ling_decode"], T=24, D=128, E=16, k=8, I=64, I_shared=64),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_matches_brute_force(name):
    cfg = SMALL[name]
    wl = generate(cfg, seed=11)
    x, wr, experts, shared = decoded(wl)
    ref = layer(x, wr, cfg.k, experts, shared, cfg.act, cfg.act_shared)
    bx, chosen, gates = brute_force_layer(x, wr, cfg.k, [experts(e) for e in range(cfg.E)],
                                          shared, cfg.act, cfg.act_shared)
    assert ref["idx"].tolist() == chosen
    g = np.take_along_axis(gates, ref["idx"].astype(np.int64), 1)
    assert np.allclose(ref["w"], g, rtol=1e-6)
    # the brute force weights are fp64 while the oracle's are stored in fp32
    assert rel_err(ref["y"], bx) < 1e-6


def test_tiny_fp32_full_size_against_brute_force():
    cfg = CONFIGS["tiny_fp32"]
    wl = generate(cfg, seed=0)
    x, wr, experts, shared = decoded(wl)
    ref = layer(x, wr, cfg.k, experts, shared, cfg.act)
    bx, chosen, _ = brute_force_layer(x, wr, cfg.k, [experts(e) for e in range(cfg.E)])
    assert ref["idx"].tolist() == chosen
    assert rel_err(ref["y"], bx) < 1e-6


def test_single_expert_top1_is_textbook_swiglu_mlp():
    """E=1, k=1: the layer is down(SiLU(gate x) * up(x)) plus the shared MLP,
    computed here with torch's own linear/silu in float64."""
    cfg = shrink(CONFIGS["qwen_decode"], T=9, D=64, E=1, k=1, I=32, I_shared=16)
    wl = generate(cfg, seed=2)
    x, wr, experts, shared = decoded(wl)
    ref = layer(x, wr, 1, experts, shared)
    w13, _, w2, _ = experts(0)
    xt = torch.tensor(x)
    gate, up = torch.tensor(w13[:32]), torch.tensor(w13[32:])
    mlp = F.linear(F.silu(F.linear(xt, gate)) * F.linear(xt, up), torch.tensor(w2))
    w13s, _, w2s, _ = shared
    sh = F.linear(F.silu(F.linear(xt, torch.tensor(w13s[:16]))) * F.linear(xt, torch.tensor(w13s[16:])),
                  torch.tensor(w2s))
    assert np.allclose(ref["w"], 1.0)
    assert rel_err(ref["y"], (mlp + sh).numpy()) < 1e-12


def test_geglu_uses_tanh_gelu_on_the_gate_half():
    rng = np.random.default_rng(3)
    X = rng.standard_normal((7, 48))
    w13 = rng.standard_normal((2 * 20, 48)) / 7
    w2 = rng.standard_normal((48, 20)) / 4.5
    o = expert_ffn(X, w13, None, w2, None, "gelu_tanh")
    xt = torch.tensor(X)
    ref = F.linear(F.gelu(F.linear(xt, torch.tensor(w13[:20])), approximate="tanh")
                   * F.linear(xt, torch.tensor(w13[20:])), torch.tensor(w2))
    assert rel_err(o, ref.numpy()) < 1e-12
    # swapping the halves gives a different answer, so the order is pinned
    sw = np.concatenate([w13[20:], w13[:20]])
    assert rel_err(expert_ffn(X, sw, None, w2, None, "gelu_tanh"), ref.numpy()) > 1e-2


def test_per_channel_scale_factors_out_of_the_reduction():
    """(A . Wq^T) * s == A . (Wq * s)^T for per-output-channel s."""
    rng = np.random.default_rng(4)
    X = rng.standard_normal((5, 64))
    q13 = rng.integers(-100, 100, (2 * 16, 64)).astype(np.float64)
    q2 = rng.integers(-100, 100, (64, 16)).astype(np.float64)
    s13 = rng.uniform(0.001, 0.01, 32)
    s2 = rng.uniform(0.001, 0.01, 64)
    a = expert_ffn(X, q13, s13, q2, s2, "silu")
    b = expert_ffn(X, q13 * s13[:, None], None, q2 * s2[:, None], None, "silu")
    assert rel_err(a, b) < 1e-13


def test_combine_of_gathered_inputs_reproduces_x():
    """combine(o := x gathered, w) = x * sum(w) = x."""
    rng = np.random.default_rng(5)
    T, E, k, D = 50, 12, 4, 16
    x = rng.standard_normal((T, D))
    idx, w = topk_softmax(rng.standard_normal((T, E)).astype(np.float32), k)
    counts, offsets, row_token, row_of_slot = permute(idx, E)
    o = x[row_token]
    y = sum(w[:, j].astype(np.float64)[:, None] * o[row_of_slot.reshape(T, k)[:, j]] for j in range(k))
    assert rel_err(y, x) < 1e-6


def test_zero_down_projection_leaves_only_the_shared_branch():
    cfg = SMALL["qwen_like"]
    wl = generate(cfg, seed=6)
    x, wr, experts, shared = decoded(wl)

    def zero_w2(e):
        w13, s13, w2, s2 = experts(e)
        return w13, s13, np.zeros_like(w2), s2
    ref = layer(x, wr, cfg.k, zero_w2, shared, cfg.act, cfg.act_shared)
    w13s, s13s, w2s, s2s = shared
    assert np.array_equal(ref["y"], expert_ffn(x, w13s, s13s, w2s, s2s, cfg.act_shared))
    only = layer(x, wr, cfg.k, experts, None, cfg.act)
    full = layer(x, wr, cfg.k, experts, shared, cfg.act, cfg.act_shared)
    assert rel_err(full["y"] - only["y"], ref["y"]) < 1e-12


def test_layer_tokens_matches_layer():
    cfg = SMALL["gemma_like"]
    wl = generate(cfg, seed=8)
    x, wr, experts, shared = decoded(wl)
    ref = layer(x, wr, cfg.k, experts, shared, cfg.act, cfg.act_shared)
    toks = [0, 5, 31]
    y = layer_tokens(toks, x, ref["idx"], ref["w"], experts, shared, cfg.act, cfg.act_shared)
    assert rel_err(y, ref["y"][toks]) < 1e-12


def test_keep_returns_consistent_intermediates():
    cfg = SMALL["qwen_like"]
    wl = generate(cfg, seed=10)
    x, wr, experts, shared = decoded(wl)
    ref = layer(x, wr, cfg.k, experts, shared, cfg.act, cfg.act_shared, keep=True)
    T, k = cfg.T, cfg.k
    y = ref["shared_out"].copy()
    for j in range(k):
        y += ref["w"][:, j].astype(np.float64)[:, None] * ref["o_perm"][ref["row_of_slot"].reshape(T, k)[:, j]]
    assert rel_err(y, ref["y"]) < 1e-14
    assert ref["h_perm"].shape == (T * k, cfg.I)
