"""Exact decoding of the stored number formats into float64.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline use this package; the library never does.

* bf16: the upper 16 bits of an IEEE-754 binary32; decoding is a 16-bit left
  shift of the raw bits.
* fp8 e4m3fn (the OCP 8-bit format the CANN Qwen3-MoE recipe quantises to,
  `float8_e4m3fn` with round-to-nearest; also the per-channel fp8 expert
  weights of the Ling-2.6-1T page, section 5): 1 sign bit, 4 exponent bits with
  bias 7, 3 mantissa bits.  Exponent field 0 encodes subnormals m * 2**-9; the
  code with all exponent and mantissa bits set (0x7F / 0xFF) is NaN; there is no
  infinity, so the largest finite magnitude is 1.75 * 2**8 = 448.
The table is built from that definition, not from any library.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode raw bf16 storage (uint16) exactly to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def fp8_e4m3fn_value(code: int) -> float:
    """Value of one e4m3fn code, straight from the format definition."""
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * man * 2.0 ** -9           # subnormal: (m/8) * 2**(1-7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


_FP8_TABLE = np.array([fp8_e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def fp8_e4m3fn_table() -> np.ndarray:
    return _FP8_TABLE.copy()


def fp8_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode raw e4m3fn storage (uint8) exactly to float64."""
    return _FP8_TABLE[np.asarray(bits, dtype=np.uint8)]


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Decode raw storage of the named format ('f32' | 'bf16' | 'fp8')."""
    if dtype == "f32":
        return np.asarray(bits, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_to_f64(bits)
    if dtype == "fp8":
        return fp8_to_f64(bits)
    raise ValueError(dtype)
