"""Pins of the oracle's dynamic per-token fp8 activation quantisation and of
its W8A8 layer (CPU only)."""
import numpy as np
import pytest

import math

from oracle.actquant import (E4M3_MAX, dequantize_rows, dequantize_subchannel, encode_e4m3fn,
                             expert_ffn_w8a8, layer_w8a8, quantize_dequantize, quantize_rows,
                             quantize_subchannel, round_bf16, rows_w8a8)
from oracle.formats import fp8_e4m3fn_table
from oracle.moe import layer, rel_err
from test_oracle_layer import decoded
from workloads import CONFIGS, generate, shrink

TABLE = fp8_e4m3fn_table()
FINITE = [c for c in range(256) if np.isfinite(TABLE[c])]


def test_every_finite_code_round_trips():
    got = encode_e4m3fn(np.array([TABLE[c] for c in FINITE], np.float32))
    want = np.array(FINITE, np.uint8)
    # +0 and -0 keep their sign bit, every other value its own code
    assert np.array_equal(got, want)


def test_midpoints_round_to_the_even_code_and_neighbours_to_the_nearest():
    pos = [c for c in range(0x7F)]
    for c in pos[:-1]:
        a, b = TABLE[c], TABLE[c + 1]
        mid = np.float32((a + b) / 2)           # exact: a and b have at most 4 significant bits
        assert float(mid) == (a + b) / 2
        even = c if c % 2 == 0 else c + 1
        assert encode_e4m3fn(np.array([mid]))[0] == even, (c, a, b)
        below = np.nextafter(mid, np.float32(-1))
        above = np.nextafter(mid, np.float32(1000))
        assert encode_e4m3fn(np.array([below]))[0] == c
        assert encode_e4m3fn(np.array([above]))[0] == c + 1


def test_saturation_and_subnormals():
    v = np.array([448.0, 449.0, 464.0, 1e6, -500.0, 2.0 ** -10, 1.5 * 2.0 ** -9,
                  2.0 ** -9, -(2.0 ** -11)], np.float32)
    got = encode_e4m3fn(v).tolist()
    # 448 = 0x7E is the largest finite code; 2**-10 is halfway between 0 and
    # the smallest subnormal (tie -> even code 0); 1.5 * 2**-9 is halfway
    # between codes 1 and 2 (tie -> 2); a tiny negative keeps its sign
    assert got == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x00, 0x02, 0x01, 0x80]


def test_random_values_round_to_a_nearest_code():
    v = (np.random.default_rng(1).standard_normal(20000) * 40).astype(np.float32)
    q = encode_e4m3fn(v)
    d = TABLE[q]
    err = np.abs(d - v.astype(np.float64))
    # no finite code is nearer than the chosen one
    others = np.abs(TABLE[np.array(FINITE)][None, :] - np.minimum(np.abs(v), 448)[:, None].astype(np.float64)
                    * np.sign(v)[:, None])
    assert np.all(err <= others.min(axis=1) + 1e-12)
    # normal range: relative error at most half an ulp (3 mantissa bits)
    normal = np.abs(v) >= 2.0 ** -6
    assert np.all(err[normal] <= np.abs(v[normal]) * 2.0 ** -4 + 1e-12)


def test_quantize_rows_scale_and_peak():
    rng = np.random.default_rng(2)
    a = rng.standard_normal((50, 96)).astype(np.float32).astype(np.float64)
    a[3] = 0.0
    q, s = quantize_rows(a)
    amax = np.abs(a).max(axis=1)
    assert s.dtype == np.float32
    assert np.array_equal(s[3:4], np.float32([1.0]))
    assert np.all(q[3] == 0)
    nz = amax > 0
    assert np.array_equal(s[nz], (amax[nz].astype(np.float32) / np.float32(448.0)))
    # each row's largest magnitude lands on the top code (+-448)
    peak = np.take_along_axis(TABLE[q], np.argmax(np.abs(a), axis=1)[:, None], 1)[:, 0]
    assert np.all(np.abs(peak[nz]) == E4M3_MAX)
    # dequantised rows within half an fp8 ulp of the row's scale grid
    d = dequantize_rows(q, s)
    assert np.all(np.abs(d - a) <= np.maximum(np.abs(a) * 2.0 ** -4, s[:, None] * 2.0 ** -10) + 1e-12)


def test_quantize_rows_is_scale_equivariant_by_powers_of_two():
    a = np.random.default_rng(3).standard_normal((20, 64)).astype(np.float32).astype(np.float64)
    q1, s1 = quantize_rows(a)
    q2, s2 = quantize_rows(a * 2.0 ** -7)
    assert np.array_equal(q1, q2)
    assert np.array_equal(s2, s1 * np.float32(2.0 ** -7))


def test_rows_on_the_fp8_grid_quantise_exactly():
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 0x7E, size=(10, 64)).astype(np.uint8)
    codes[:, 0] = 0x7E                                  # peak 448 -> scale 1 after x 2**-3
    signs = rng.integers(0, 2, size=codes.shape).astype(np.uint8) << 7
    codes |= signs
    a = TABLE[codes] * 2.0 ** -3
    q, s = quantize_rows(a)
    assert np.array_equal(s, np.full(10, 2.0 ** -3, np.float32))
    assert np.array_equal(TABLE[q], TABLE[codes])


def test_round_bf16_matches_bit_truncation_rules():
    v = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20, -2.5], np.float64)
    # ties go to the even bf16 mantissa; anything above the tie rounds up
    assert round_bf16(v).tolist() == [1.0, 1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7, -2.5]


W8A8 = {
    "ling_fp8": shrink(CONFIGS["ling_decode"], T=24, D=128, E=16, k=8, I=64, I_shared=64),
    "ling_prefill_like": shrink(CONFIGS["ling_prefill"], T=40, D=256, E=8, k=4, I=128, I_shared=128),
}


@pytest.mark.parametrize("name", list(W8A8))
def test_w8a8_layer_is_close_to_the_plain_definition(name):
    """The W8A8 layer differs from the exact one only by the activation
    quantisation: a few per cent of the output's range, never more."""
    cfg = W8A8[name]
    x, wr, experts, shared = decoded(generate(cfg, seed=5))
    ref = layer(x, wr, cfg.k, experts, shared, cfg.act, cfg.act_shared)
    q = layer_w8a8(x, wr, cfg.k, experts, shared, cfg.act, cfg.act_shared)
    for n in ("idx", "counts", "offsets", "row_token", "row_of_slot"):
        assert np.array_equal(np.asarray(q[n]), np.asarray(ref[n]))
    err = rel_err(q["y"], ref["y"])
    assert 1e-4 < err < 0.08, err


def test_token_by_token_evaluation_matches_the_whole_layer():
    cfg = W8A8["ling_prefill_like"]
    x, wr, experts, shared = decoded(generate(cfg, seed=7))
    q = layer_w8a8(x, wr, cfg.k, experts, shared, cfg.act, cfg.act_shared)
    toks = [0, 5, 17, 39]
    y = rows_w8a8(toks, x, q["idx"], q["w"], experts, shared, cfg.act, cfg.act_shared)
    assert np.allclose(y, q["y"][toks], rtol=1e-12, atol=1e-12)


# ---- the sub-channel variant ("Qwen 3.5 MoE on Ironwood" page, MoE track, GMM
# v2: fp8 activations with one scale per 512-element sub-channel)

def test_subchannel_with_one_slice_is_the_per_row_rule():
    a = np.random.default_rng(11).standard_normal((30, 512)).astype(np.float32).astype(np.float64)
    a[4] = 0.0
    q1, s1 = quantize_subchannel(a, 512)
    q2, s2 = quantize_rows(a)
    assert np.array_equal(q1, q2) and np.array_equal(s1[:, 0], s2)


def test_subchannel_hand_example():
    """A row of two slices worked by hand: slice 0 peaks at 896 (scale 2),
    slice 1 at 0.875 (scale 0.875 / 448 = 2^-9); each element's code is taken
    against its own slice's scale."""
    a = np.zeros((1, 1024))
    a[0, 0], a[0, 1], a[0, 2] = 896.0, 1.0, -2.0
    a[0, 512], a[0, 513] = 0.875, 0.4375
    q, s = quantize_subchannel(a, 512)
    assert s.tolist() == [[2.0, 2.0 ** -9]]
    # 448 -> 0x7E; 0.5 = 2^-1 -> exponent field 6, mantissa 0 -> 0x30;
    # -1 -> 0xB8; 224 = 1.75 * 2^7 -> exponent field 14, mantissa 6 -> 0x76
    assert q[0, :3].tolist() == [0x7E, 0x30, 0xB8]
    assert q[0, 512:514].tolist() == [0x7E, 0x76]
    assert np.all(q[0, 3:512] == 0) and np.all(q[0, 514:] == 0)
    # with one scale for the row, the second slice would sit on the coarse
    # grid of scale 2: 0.875 / 2 = 0.4375 = 1.75 * 2^-2 -> 0x2E
    qr, sr = quantize_rows(a)
    assert sr.tolist() == [2.0] and qr[0, 512] == 0x2E


@pytest.mark.parametrize("col,expect", [(511, [100.0, 1.0, 1.0]), (512, [1.0, 100.0, 1.0]),
                                        (1023, [1.0, 100.0, 1.0]), (1024, [1.0, 1.0, 100.0])])
def test_subchannel_slice_boundaries(col, expect):
    a = np.ones((2, 1536))
    a[1, col] = 100.0
    _, s = quantize_subchannel(a, 512)
    assert np.array_equal(s[0], np.full(3, np.float32(1.0) / np.float32(448.0), np.float32))
    want = np.array(expect, np.float32) / np.float32(448.0)
    assert np.array_equal(s[1], want)


def test_subchannel_error_is_bounded_by_each_slices_own_scale():
    """Rows whose slices differ in magnitude by up to 2^16: every element
    stays within half an fp8 ulp of its own slice's grid, while one scale per
    row puts the small slices below the fp8 subnormals (2^-9 of the scale)."""
    rng = np.random.default_rng(12)
    b = rng.integers(0, 2, size=(16, 4))
    b[:, 0] = 0                                            # every row has a large slice
    mags = 2.0 ** (rng.integers(-3, 4, size=(16, 1)) - 16 * b)
    a = (rng.standard_normal((16, 2048)) * np.repeat(mags, 512, axis=1)).astype(np.float32).astype(np.float64)
    q, s = quantize_subchannel(a, 512)
    d = dequantize_subchannel(q, s)
    srep = np.repeat(s.astype(np.float64), 512, axis=1)
    assert np.all(np.abs(d - a) <= np.maximum(np.abs(a) * 2.0 ** -4, srep * 2.0 ** -10) + 1e-15)
    # each slice's largest magnitude lands on the top code
    for j in range(4):
        blk = a[:, 512 * j:512 * (j + 1)]
        peak = np.take_along_axis(TABLE[q[:, 512 * j:512 * (j + 1)]], np.argmax(np.abs(blk), axis=1)[:, None], 1)
        assert np.all(np.abs(peak) == E4M3_MAX)
    # the slices 2^16 below their row's large ones: relative error per slice
    dr = dequantize_rows(*quantize_rows(a))
    small = b == 1
    assert small.sum() >= 8
    for r, j in zip(*np.nonzero(small)):
        blk = slice(512 * j, 512 * (j + 1))
        e_sub = np.abs(d[r, blk] - a[r, blk]).sum() / np.abs(a[r, blk]).sum()
        e_row = np.abs(dr[r, blk] - a[r, blk]).sum() / np.abs(a[r, blk]).sum()
        assert e_sub < 0.04 and e_row > 0.1, (r, j, e_sub, e_row)


def test_subchannel_expert_hand_case():
    """One token through one expert, worked by hand.  x: slice 0 all 7
    (scale 7 / 448 = 2^-6), slice 1 all 0.01 (scale 0.01 / 448); the gate and
    up rows read slice 1 only (gate: mean, up: sum), so g = 0.01 and u = 5.12
    up to the slice's quantisation, h = bf16(silu(g) u) on all 512 columns, and
    a down row of 1 / 512 returns h.  One scale for the whole row would give
    g = 0.009765625, u = 5.0 (0.01 * 64 = 0.64 -> 0.625 on the fp8 grid)."""
    D, I = 1024, 512
    x = np.concatenate([np.full(512, 7.0), np.full(512, np.float32(0.01))])[None, :]
    ind = np.concatenate([np.zeros(512), np.ones(512)])
    w13 = np.vstack([np.tile(ind / 512.0, (I, 1)), np.tile(ind, (I, 1))])
    w2 = np.full((3, I), 1.0 / 512.0)
    silu = lambda z: z / (1.0 + math.exp(-z))
    for width, g, u in ((512, 0.01, 5.12), (None, 0.009765625, 5.0)):
        xd = quantize_dequantize(x, width)
        o = expert_ffn_w8a8(xd, w13, None, w2, None, "silu", width)
        h = float(round_bf16(np.array([silu(g) * u]))[0])
        assert np.allclose(o, h, rtol=2e-3), (width, o[0, 0], h)
    assert abs(round_bf16(np.array([silu(0.01) * 5.12]))[0] - round_bf16(np.array([silu(0.009765625) * 5.0]))[0]) > 1e-3


def test_subchannel_rejects_ragged_rows():
    with pytest.raises(ValueError):
        quantize_subchannel(np.ones((2, 700)), 512)


W8A8_SUB = {
    "ling_prefill_like": shrink(CONFIGS["ling_prefill"], T=40, D=1024, E=8, k=4, I=512, I_shared=512),
}


def test_subchannel_layer_is_close_to_the_plain_definition_and_evaluates_token_by_token():
    cfg = W8A8_SUB["ling_prefill_like"]
    x, wr, experts, shared = decoded(generate(cfg, seed=13))
    ref = layer(x, wr, cfg.k, experts, shared, cfg.act, cfg.act_shared)
    q = layer_w8a8(x, wr, cfg.k, experts, shared, cfg.act, cfg.act_shared, width=512)
    assert np.array_equal(q["idx"], ref["idx"])
    assert q["x_scales"].shape == (cfg.T, cfg.D // 512)
    err = rel_err(q["y"], ref["y"])
    assert 1e-4 < err < 0.08, err
    toks = [0, 9, 39]
    y = rows_w8a8(toks, x, q["idx"], q["w"], experts, shared, cfg.act, cfg.act_shared, width=512)
    assert np.allclose(y, q["y"][toks], rtol=1e-12, atol=1e-12)
