"""Pins of the oracle's number-format decoding (CPU only)."""
import math

import numpy as np
import pytest
import torch

from oracle.formats import bf16_to_f64, fp8_e4m3fn_table, fp8_to_f64
from workloads.gen import _quant_fp8_rows


def test_fp8_table_matches_library_on_all_codes():
    """All 256 codes against torch's float8_e4m3fn -> float64 conversion."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    lib = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = fp8_e4m3fn_table()
    nan_l, nan_o = np.isnan(lib), np.isnan(ours)
    assert np.array_equal(nan_l, nan_o)
    assert np.array_equal(lib[~nan_l], ours[~nan_o])
    # the sign of zero is part of the format
    assert np.array_equal(np.signbit(lib[~nan_l]), np.signbit(ours[~nan_o]))


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0x40, 2.0), (0x3C, 1.5), (0x7E, 448.0), (0xFE, -448.0),
    (0x77, 240.0), (0xB8, -1.0),
])
def test_fp8_known_codes(code, value):
    """Values fixed by the e4m3fn definition (bias 7, no infinity, max 448)."""
    assert fp8_to_f64(np.array([code], np.uint8))[0] == value


def test_fp8_nan_and_negative_zero():
    t = fp8_e4m3fn_table()
    assert math.isnan(t[0x7F]) and math.isnan(t[0xFF])
    assert np.sum(np.isnan(t)) == 2
    assert t[0x80] == 0.0 and math.copysign(1.0, t[0x80]) == -1.0
    finite = t[~np.isnan(t)]
    assert finite.max() == 448.0 and finite.min() == -448.0


def test_fp8_every_code_exact_in_bf16():
    """Every finite e4m3fn value is a bf16 value (8-bit exponent, 7-bit
    mantissa), which is what lets W8A16 decode the weights exactly."""
    t = fp8_e4m3fn_table()
    f = t[~np.isnan(t)]
    as_bf16 = torch.tensor(f, dtype=torch.float64).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(as_bf16, f)


def test_bf16_decode_matches_library():
    g = torch.Generator().manual_seed(3)
    v = torch.randn(4096, generator=g) * 100
    v = torch.cat([v, torch.tensor([0.0, -0.0, 1e-40, -3.4e38, 65504.0])])
    b = v.to(torch.bfloat16)
    lib = b.to(torch.float64).numpy()
    ours = bf16_to_f64(b.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(lib, ours)
    assert np.array_equal(np.signbit(lib), np.signbit(ours))


def test_generator_fp8_quantiser_properties():
    """Per-row scales s = amax/448; the row maximum lands on +-448; decoded
    values are within half a unit in the last place (RNE) of W/s."""
    g = torch.Generator().manual_seed(5)
    w = torch.randn(64, 256, generator=g) / 16
    q, s = _quant_fp8_rows(w)
    qd = fp8_to_f64(q.view(torch.uint8).numpy())
    ref = (w.double() / s.double()[:, None]).numpy()
    amax_pos = np.argmax(np.abs(ref), axis=1)
    assert np.all(np.abs(qd[np.arange(64), amax_pos]) == 448.0)
    # half-ulp bound: normals have 3 mantissa bits, subnormal spacing 2^-9
    ulp = np.where(np.abs(qd) >= 2.0 ** -6,
                   2.0 ** (np.floor(np.log2(np.maximum(np.abs(qd), 1e-300))) - 3), 2.0 ** -9)
    assert np.all(np.abs(qd - ref) <= ulp / 2 + 1e-12)
    assert np.allclose(s.numpy(), np.abs(w.numpy()).max(axis=1) / 448.0, rtol=1e-7)
