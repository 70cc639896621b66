"""Pins of the oracle's dynamic per-token fp8 activation quantisation and of
its W8A8 layer (CPU only)."""
import numpy as np
import pytest

from oracle.actquant import (E4M3_MAX, dequantize_rows, encode_e4m3fn, layer_w8a8,
                             quantize_rows, round_bf16, rows_w8a8)
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
