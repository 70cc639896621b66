"""Pins of the quantised-mode steps of the oracle (CPU only), each against an
independent evaluation that a plausible slip in the oracle would fail:

* decode_mxfp4_weight: hand-packed bytes and E8M0 scales with known values
  (nibble order and the [K/128][N][4] scale layout of the stored MXFP4 weight),
  and the round trip of the input generator's MXFP4 quantiser within half an
  e2m1 step times the block scale;
* expert_ffn_w8a8 / expert_ffn_w4a8: a one-row, one-expert case evaluated
  step by step with scalar Python arithmetic and torch's own float8 cast, in
  the order the "Ling-2.6-1T with SGLang-JAX" page (section 5, activation
  quantisation) and the "CANN Qwen3-MoE" page (W4A8 compute decomposition)
  imply for the down projection's input: h is stored in bf16 and the stored
  value is quantised.  The same case also shows that skipping the bf16
  rounding, or quantising h before it, moves the result;
* rel_err: the max-over-tensor relative error on hand-made arrays.
"""
import math
import struct

import numpy as np
import pytest
import torch

from oracle.actquant import expert_ffn_w8a8
from oracle.moe import rel_err
from oracle.mx import decode_mxfp4_weight, expert_ffn_w4a8
from workloads.gen import _quant_mxfp4

# e2m1 magnitudes by code (sign bit 0x8), straight from the format: 1 sign,
# 2 exponent bits (bias 1), 1 mantissa bit, exponent 0 subnormal (0.5 * m)
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def e2m1(code: int) -> float:
    v = E2M1[code & 7]
    return -v if code & 8 else v


def f32(v: float) -> float:
    return struct.unpack("<f", struct.pack("<f", v))[0]


def bf16(v: float) -> float:
    """float -> float32 -> bf16, round to nearest even, as a float."""
    (b,) = struct.unpack("<I", struct.pack("<f", v))
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return struct.unpack("<f", struct.pack("<I", b))[0]


def fp8_torch(v: float) -> float:
    """Nearest e4m3fn value (ties to even) by torch's float8 cast."""
    assert abs(v) <= 448.0
    return float(torch.tensor([v], dtype=torch.float32).to(torch.float8_e4m3fn).to(torch.float64)[0])


def silu(z: float) -> float:
    return z / (1.0 + math.exp(-z))


# ------------------------------------------------------------------ MXFP4 weights
def test_decode_mxfp4_weight_hand_packed():
    N, K = 2, 256
    codes = [[(n * 37 + k * 5 + (k // 3)) % 16 for k in range(K)] for n in range(N)]
    # distinct E8M0 codes for every (128-group, row, 32-block)
    sc = np.array([[[118 + 8 * g + 4 * n + b for b in range(4)] for n in range(N)] for g in range(K // 128)],
                  np.uint8)
    packed = np.array([[codes[n][2 * j] | (codes[n][2 * j + 1] << 4) for j in range(K // 2)] for n in range(N)],
                      np.uint8)
    want = np.array([[e2m1(codes[n][k]) * 2.0 ** (int(sc[k // 128, n, (k % 128) // 32]) - 127) for k in range(K)]
                     for n in range(N)])
    got = decode_mxfp4_weight(packed, sc)
    assert got.shape == (N, K)
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))
    # the pin has power: the other nibble order, or the scales read as
    # [N][K/128][4], give other values
    swapped = ((packed & 0xF) << 4) | (packed >> 4)
    assert not np.array_equal(decode_mxfp4_weight(swapped, sc), want)
    assert not np.array_equal(decode_mxfp4_weight(packed, sc.transpose(1, 0, 2).copy()), want)


def test_mxfp4_weight_round_trip_within_half_a_step():
    g = torch.Generator().manual_seed(11)
    w = torch.randn(24, 384, generator=g) * torch.exp2(torch.randint(-6, 6, (24, 1), generator=g).float())
    w[3, 32:64] = 0.0
    packed, sc = _quant_mxfp4(w)
    d = decode_mxfp4_weight(packed.numpy(), sc.numpy())
    w64 = w.numpy().astype(np.float64)
    blocks = np.abs(w64).reshape(24, 12, 32)
    amax = blocks.max(axis=2)
    scale = np.where(amax > 0, np.exp2(np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2), 2.0 ** -127)
    m = blocks / scale[:, :, None]                     # scaled magnitudes, below 8
    half = np.where(m < 2, 0.25, np.where(m < 4, 0.5, 1.0))
    bound = np.where(m <= 6, half, m - 6) * scale[:, :, None]
    err = np.abs(d - w64).reshape(24, 12, 32)
    assert np.all(err <= bound)
    assert np.all(d[3, 32:64] == 0)


# ------------------------------------------------------------------ quantised expert FFNs
def _w8a8_case():
    # x on the fp8 grid of its own row scale: codes 448, -224, 112, 0 with s = fl32(1/448)
    x = np.array([[1.0, -0.5, 0.25, 0.0]])
    g = [1.3, -0.7]
    u = [0.9, 2.1]
    w13 = np.zeros((4, 4))
    w13[:, 0] = g + u
    w13[:, 1] = [0.25, 0.5, -0.125, 0.0]
    s13 = np.array([2.0, 1.0, 0.5, 1.0])
    w2 = np.array([[1.0, 0.0], [0.0, 1.0], [0.5, 0.25], [0.0, 0.0]])
    s2 = np.array([1.0, 2.0, 1.0, 1.0])
    return x, w13, s13, w2, s2


def _w8a8_chain(x, w13, s13, w2, s2, bf16_h=True, quant_first=False):
    """The W8A8 expert step by step in scalar arithmetic (fp32 where the
    quantiser works in fp32, float64 otherwise)."""
    sx = f32(f32(float(np.abs(x).max())) / f32(448.0))
    xd = [fp8_torch(f32(f32(v) / sx)) * sx for v in x[0]]
    gu = [sum(xd[d] * w13[n, d] for d in range(4)) * s13[n] for n in range(4)]
    h = [silu(gu[i]) * gu[2 + i] for i in range(2)]

    def quant(row):
        s = f32(f32(max(abs(v) for v in row)) / f32(448.0))
        return [fp8_torch(f32(f32(v) / s)) * s for v in row]
    if quant_first:
        hd = [bf16(v) for v in quant(h)]
    else:
        hd = quant([bf16(v) for v in h] if bf16_h else h)
    return np.array([[sum(hd[i] * w2[n, i] for i in range(2)) * s2[n] for n in range(4)]])


def test_expert_ffn_w8a8_one_row_by_hand():
    x, w13, s13, w2, s2 = _w8a8_case()
    sx = np.float32(1.0) / np.float32(448.0)
    xd = np.array([[448.0, -224.0, 112.0, 0.0]]) * float(sx)     # the row's fp8 dequantisation
    got = expert_ffn_w8a8(xd, w13, s13, w2, s2, "silu")
    want = _w8a8_chain(x, w13, s13, w2, s2)
    assert np.allclose(got, want, rtol=1e-13, atol=0), (got, want)
    # the case tells the mistakes apart from the definition
    for bad in (_w8a8_chain(x, w13, s13, w2, s2, bf16_h=False),
                _w8a8_chain(x, w13, s13, w2, s2, quant_first=True)):
        assert rel_err(bad, want) > 1e-5


def _w4a8_case():
    rng = np.random.default_rng(21)
    D, I = 4, 32
    xd = np.array([[1.0, -0.75, 0.5, 0.125]])
    w13 = rng.standard_normal((2 * I, D)) * 0.6
    w2 = rng.standard_normal((D, I)) * 0.2
    return xd, w13, w2


def _w4a8_chain(xd, w13, w2, bf16_h=True, quant_first=False):
    I = w13.shape[0] // 2
    gu = [float(sum(xd[0, d] * w13[n, d] for d in range(xd.shape[1]))) for n in range(2 * I)]
    h = [silu(gu[i]) * gu[I + i] for i in range(I)]

    def quant(row):                  # one MXFP8 block of 32: E8M0 scale 2**(floor(log2 amax) - 8)
        amax = max(abs(v) for v in row)
        _, e = math.frexp(amax)      # amax = m * 2**e, m in [0.5, 1)
        sc = 2.0 ** (e - 1 - 8)
        return [fp8_torch(v / sc) * sc for v in row]
    if quant_first:
        hd = [bf16(v) for v in quant(h)]
    else:
        hd = quant([bf16(v) for v in h] if bf16_h else h)
    return np.array([[sum(hd[i] * w2[n, i] for i in range(I)) for n in range(w2.shape[0])]])


def test_expert_ffn_w4a8_one_row_by_hand():
    xd, w13, w2 = _w4a8_case()
    got = expert_ffn_w4a8(xd, w13, w2, "silu")
    want = _w4a8_chain(xd, w13, w2)
    assert np.allclose(got, want, rtol=1e-13, atol=1e-15), (got, want)
    for bad in (_w4a8_chain(xd, w13, w2, bf16_h=False), _w4a8_chain(xd, w13, w2, quant_first=True)):
        assert rel_err(bad, want) > 1e-5


# ------------------------------------------------------------------ the parity metric
def test_rel_err_is_max_abs_diff_over_max_abs_ref():
    ref = np.array([[1.0, -4.0], [2.0, 0.5]])
    got = ref + np.array([[0.0, 0.1], [-0.2, 0.0]])
    assert rel_err(got, ref) == pytest.approx(0.2 / 4.0, rel=1e-15)
    assert rel_err(-ref, ref) == pytest.approx(8.0 / 4.0, rel=1e-15)
    assert rel_err(ref, ref) == 0.0
    # over the whole tensor, not per element: a small element's relative error
    # does not dominate
    assert rel_err(np.array([1000.0, 2e-6]), np.array([1000.0, 1e-6])) == pytest.approx(1e-9, rel=1e-9)
    # a zero reference gives the absolute error; empty tensors give 0
    assert rel_err(np.array([0.5, -0.25]), np.zeros(2)) == 0.5
    assert rel_err(np.zeros((0, 3)), np.zeros((0, 3))) == 0.0
    # bf16 storage is compared after exact upcast (float32 input accepted as is)
    assert rel_err(np.float32([1.5]), np.array([1.0])) == 0.5
