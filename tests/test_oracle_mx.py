"""Pins of the oracle's microscaling (MX) formats and of its W4A8 layer (CPU only)."""
import numpy as np
import pytest

from oracle.formats import fp8_e4m3fn_table
from oracle.moe import layer, rel_err
from oracle.mx import (e8m0_value, fp4_e2m1_table, layer_w4a8, mx_dequantize, mx_quantize,
                       mx_round_trip, rows_w4a8)
from test_oracle_layer import decoded
from workloads import CONFIGS, generate, shrink

E2M1 = fp4_e2m1_table()
E4M3 = fp8_e4m3fn_table()


def test_e2m1_table_from_the_format():
    # 0, 0.5 (subnormal), then 1, 1.5, 2, 3, 4, 6 and their negatives
    assert E2M1[:8].tolist() == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert E2M1[8:].tolist() == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    assert np.signbit(E2M1[8])


def test_e8m0_scale_values():
    assert e8m0_value(np.array([127, 128, 0, 254])).tolist() == [1.0, 2.0, 2.0 ** -127, 2.0 ** 127]


@pytest.mark.parametrize("fmt,table,emax,vmax", [("e2m1", E2M1, 2, 6.0), ("e4m3", E4M3, 8, 448.0)])
def test_block_exponent_and_saturation(fmt, table, emax, vmax):
    rng = np.random.default_rng(0)
    a = rng.standard_normal((6, 64)) * np.exp2(rng.integers(-10, 10, size=(6, 1)))
    a[2, :32] = 0.0                                 # a block of zeros
    q, s = mx_quantize(a, fmt)
    amax = np.abs(a.reshape(6, 2, 32)).max(axis=2)
    nz = amax > 0
    # the scale exponent is floor(log2 amax) - emax
    assert np.array_equal(s[nz].astype(int) - 127, np.floor(np.log2(amax[nz])).astype(int) - emax)
    assert s[2, 0] == 0 and np.all(q[2, :32] & (0x7 if fmt == "e2m1" else 0x7F) == 0)
    # scaled magnitudes are below 2**(emax+1); beyond the largest payload they saturate
    d = table[q].reshape(6, 2, 32)
    assert np.all(np.abs(d) <= vmax)
    scaled = np.abs(a.reshape(6, 2, 32)) / e8m0_value(s)[:, :, None]
    assert np.all(scaled < 2.0 ** (emax + 1))
    assert np.all(np.abs(d)[scaled >= vmax] == vmax)


@pytest.mark.parametrize("fmt", ["e2m1", "e4m3"])
def test_nearest_even_rounding_of_scaled_values(fmt):
    table = E2M1 if fmt == "e2m1" else E4M3
    vmax = 6.0 if fmt == "e2m1" else 448.0
    pos = np.array(sorted(set(np.abs(table[np.isfinite(table)]).tolist())))
    # one block whose peak fixes the scale at 2**0 (peak in [2**emax, 2**(emax+1))),
    # the other entries are midpoints between neighbouring payload values
    mids = (pos[:-1] + pos[1:]) / 2
    emax = 2 if fmt == "e2m1" else 8
    blk = np.zeros(32)
    blk[0] = 2.0 ** emax
    n = min(31, len(mids))
    blk[1:1 + n] = mids[:n]
    q, s = mx_quantize(blk[None, :], fmt)
    assert s[0, 0] == 127
    got = np.abs(table[q[0, 1:1 + n]])
    codes = np.arange(len(pos))
    for i in range(n):
        lo, hi = i, i + 1          # mids[i] lies between pos[lo] and pos[hi]
        # ties go to the value whose code is even (code = rank among magnitudes)
        want = pos[lo] if codes[lo] % 2 == 0 else pos[hi]
        assert got[i] == want, (i, mids[i], got[i], want)


@pytest.mark.parametrize("fmt", ["e2m1", "e4m3"])
def test_round_trip_error_bound_and_grid_values(fmt):
    rng = np.random.default_rng(1)
    a = rng.standard_normal((20, 128))
    d = mx_round_trip(a, fmt)
    blocks = np.abs(a).reshape(20, 4, 32).max(axis=2)
    # error at most half a step of the element grid at the block's top binade,
    # except for magnitudes beyond the largest payload, which saturate to it
    mbits, vmax, emax = (1, 6.0, 2) if fmt == "e2m1" else (3, 448.0, 8)
    f = np.floor(np.log2(blocks))
    step = np.exp2(f - mbits)[:, :, None]
    scale = np.exp2(f - emax)[:, :, None]
    a3, d3 = a.reshape(20, 4, 32), d.reshape(20, 4, 32)
    sat = np.abs(a3) > vmax * scale
    assert np.all(np.abs(d3 - a3)[~sat] <= (step / 2 + 0 * a3)[~sat])
    assert np.array_equal(np.abs(d3[sat]), (vmax * scale + 0 * a3)[sat])
    # values already on a block grid with the right peak come back unchanged
    assert np.array_equal(mx_round_trip(d, fmt), d)


W4A8 = {"ling_like": shrink(CONFIGS["ling_decode"], T=24, D=128, E=16, k=8, I=128, I_shared=128,
                            w_dtype="mxfp4", shared_w_dtype="mxfp4")}


def test_w4a8_layer_keeps_routing_and_stays_close_to_the_exact_layer():
    cfg = W4A8["ling_like"]
    x, wr, experts, shared = decoded(generate(cfg, seed=5))
    ref = layer(x, wr, cfg.k, experts, shared, cfg.act, cfg.act_shared)
    q = layer_w4a8(x, wr, cfg.k, experts, shared, cfg.act, cfg.act_shared)
    for n in ("idx", "counts", "offsets", "row_token", "row_of_slot"):
        assert np.array_equal(np.asarray(q[n]), np.asarray(ref[n]))
    err = rel_err(q["y"], ref["y"])
    # the weights are the same decoded MXFP4 values on both sides: only the
    # MXFP8 activations differ
    assert 1e-4 < err < 0.08, err
    toks = [0, 7, 23]
    y = rows_w4a8(toks, x, q["idx"], q["w"], experts, shared, cfg.act, cfg.act_shared)
    assert np.allclose(y, q["y"][toks], rtol=1e-12, atol=1e-12)


def test_generator_mxfp4_matches_the_oracle_quantiser():
    """The input generator's MXFP4 weights (torch) are the oracle's MX
    quantisation (NumPy) of the same fp32 draws, codes and scales alike."""
    import torch
    from workloads.gen import _quant_mxfp4
    g = torch.Generator().manual_seed(3)
    w = torch.randn(48, 256, generator=g) * 0.05
    w[5, :32] = 0.0
    packed, sc = _quant_mxfp4(w)
    codes, scales = mx_quantize(w.numpy().astype(np.float64), "e2m1")
    p = packed.numpy()
    assert np.array_equal(p & 0xF, codes[:, 0::2]) and np.array_equal(p >> 4, codes[:, 1::2])
    assert np.array_equal(sc.numpy().transpose(1, 0, 2).reshape(48, -1), scales)
