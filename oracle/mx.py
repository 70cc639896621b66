"""Microscaling (MX) block formats and the W4A8 layer.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline use this module; the HIP library never does, and the two share no code.

The "CANN Qwen3-MoE" page (high-throughput prefill: the W4A8 compute
decomposition) runs the MoE with MXFP4 weights and activations quantised
dynamically to MXFP8 (an e4m3fn payload with a per-block scale) before the
grouped matmul.  The page does not spell the formats out; the readings here
are those of the Open Compute Project microscaling formats:

  * a block is 32 consecutive elements along the reduction (K) dimension of a
    row, sharing one E8M0 scale: 8 exponent bits, bias 127, value 2**(e-127);
  * element payloads: e2m1 (MXFP4: sign, 2 exponent bits with bias 1, 1
    mantissa bit; exponent field 0 is the subnormal 0.5 * m; magnitudes 0,
    0.5, 1, 1.5, 2, 3, 4, 6) or e4m3fn (MXFP8, oracle.formats);
  * quantising a block: shared exponent floor(log2(max |v|)) - emax, where
    emax is the element format's largest exponent (2 for e2m1, 8 for e4m3fn),
    clamped to [-127, 127] (a block of zeros gets -127); elements are the
    nearest payload values of v / 2**shared (an exact power-of-two division),
    ties to the even code, magnitudes beyond the format's largest saturating
    to it.

The layer (W4A8): routing exactly as the plain layer on the bf16 activations;
x is quantised to MXFP8 per token and per block, the expert GEMMs multiply the
decoded blocks (float64), h is stored in bf16 and quantised the same way
before the down projection.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .actquant import round_bf16
from .formats import fp8_e4m3fn_table
from .moe import ACTS, permute, router_logits, topk_softmax

BLOCK = 32
_E4M3 = fp8_e4m3fn_table()


def fp4_e2m1_value(code: int) -> float:
    """Value of one e2m1 code from the format definition."""
    sign = -1.0 if code & 0x8 else 1.0
    exp = (code >> 1) & 0x3
    man = code & 0x1
    if exp == 0:
        return sign * 0.5 * man
    return sign * (1.0 + 0.5 * man) * 2.0 ** (exp - 1)


_E2M1 = np.array([fp4_e2m1_value(c) for c in range(16)], dtype=np.float64)


def fp4_e2m1_table() -> np.ndarray:
    return _E2M1.copy()


def e8m0_value(e: np.ndarray) -> np.ndarray:
    """2**(e - 127) for E8M0 codes (255, the NaN code, is outside the contract)."""
    return np.exp2(np.asarray(e, np.float64) - 127.0)


# element formats: (decode table, largest exponent, largest magnitude, codes of the
# non-negative values in increasing order)
_FORMATS = {
    "e2m1": (_E2M1, 2, 6.0, np.arange(8)),
    "e4m3": (_E4M3, 8, 448.0, np.arange(0x7F)),
}


def _encode(v: np.ndarray, fmt: str) -> np.ndarray:
    """Nearest payload code of each value (ties to the even code, saturating)."""
    table, _, vmax, pos = _FORMATS[fmt]
    vals = table[pos]
    v = np.asarray(v, np.float64)
    mag = np.minimum(np.abs(v), vmax)
    hi = np.clip(np.searchsorted(vals, mag, side="left"), 0, len(vals) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = mag - vals[lo], vals[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (pos[hi] % 2 == 0))
    code = np.where(pick_hi, pos[hi], pos[lo]).astype(np.uint8)
    sign_bit = 0x8 if fmt == "e2m1" else 0x80
    return np.where(np.signbit(v), code | sign_bit, code).astype(np.uint8)


def mx_quantize(a: np.ndarray, fmt: str):
    """Rows [n, K] (K a multiple of 32) -> (codes uint8 [n, K], E8M0 scales uint8 [n, K/32])."""
    a = np.asarray(a, np.float64)
    n, K = a.shape
    assert K % BLOCK == 0
    blocks = a.reshape(n, K // BLOCK, BLOCK)
    amax = np.abs(blocks).max(axis=2)
    _, emax, _, _ = _FORMATS[fmt]
    # floor(log2 amax) from the exponent, exactly: amax = m * 2**p with m in [0.5, 1)
    _, p = np.frexp(amax)
    shared = np.where(amax > 0, p - 1, -127) - emax
    shared = np.clip(shared, -127, 127).astype(np.int64)
    codes = _encode(blocks / np.exp2(shared)[:, :, None], fmt).reshape(n, K)
    return codes, (shared + 127).astype(np.uint8)


def mx_dequantize(codes: np.ndarray, scales: np.ndarray, fmt: str) -> np.ndarray:
    table = _FORMATS[fmt][0]
    codes = np.asarray(codes, np.uint8)
    n, K = codes.shape
    v = table[codes].reshape(n, K // BLOCK, BLOCK) * e8m0_value(scales)[:, :, None]
    return v.reshape(n, K)


def mx_round_trip(a: np.ndarray, fmt: str) -> np.ndarray:
    return mx_dequantize(*mx_quantize(a, fmt), fmt)


def decode_mxfp4_weight(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Stored MXFP4 weight -> float64 [N, K]: packed [N, K/2] (element 2j in the
    low nibble), scales [K/128, N, 4] (per group of 128 K elements, each row's
    four block scales side by side)."""
    packed = np.asarray(packed, np.uint8)
    N, K2 = packed.shape
    codes = np.empty((N, 2 * K2), np.uint8)
    codes[:, 0::2] = packed & 0xF
    codes[:, 1::2] = packed >> 4
    sc = np.asarray(scales, np.uint8).transpose(1, 0, 2).reshape(N, -1)     # [N, K/32]
    return mx_dequantize(codes, sc, "e2m1")


def decode_weight(bits: np.ndarray, scales, dtype: str):
    """(decoded float64 weight, per-output-channel scale or None) of a stored
    expert matrix in any of the weight formats."""
    if dtype == "mxfp4":
        return decode_mxfp4_weight(bits, scales), None
    from .formats import decode
    return decode(bits, dtype), scales


def expert_ffn_w4a8(Xd: np.ndarray, w13: np.ndarray, w2: np.ndarray, act: str) -> np.ndarray:
    """One gated expert on MXFP8-dequantised rows Xd with decoded MXFP4
    weights w13 [2I, D] and w2 [D, I]: h is stored in bf16 and quantised to
    MXFP8 before the down projection."""
    I = w13.shape[0] // 2
    gu = Xd @ w13.T
    h = round_bf16(ACTS[act](gu[:, :I]) * gu[:, I:])
    return mx_round_trip(h, "e4m3") @ w2.T


def layer_w4a8(x: np.ndarray, wr: np.ndarray, k: int, expert, shared: Optional[tuple] = None,
               act: str = "silu", act_shared: str = "silu",
               logits_in: Optional[np.ndarray] = None, renormalize: bool = True) -> dict:
    """The layer with MXFP4 weights and MXFP8 activations.  expert(e) returns
    the decoded (w13, None, w2, None); shared likewise or None."""
    x = np.asarray(x, np.float64)
    T, D = x.shape
    E = wr.shape[0]
    logits = router_logits(x, wr) if logits_in is None else np.asarray(logits_in, np.float32)
    idx, w = topk_softmax(logits, k, renormalize)
    counts, offsets, row_token, row_of_slot = permute(idx, E)
    xd = mx_round_trip(x, "e4m3")
    o_perm = np.zeros((T * k, D), dtype=np.float64)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        w13, _, w2, _ = expert(e)
        o_perm[r0:r1] = expert_ffn_w4a8(xd[row_token[r0:r1]], w13, w2, act)
    y = np.zeros((T, D), dtype=np.float64)
    for j in range(k):
        y += w[:, j].astype(np.float64)[:, None] * o_perm[row_of_slot.reshape(T, k)[:, j]]
    if shared is not None:
        y += expert_ffn_w4a8(xd, shared[0], shared[2], act_shared)
    return dict(y=y, logits=logits, idx=idx, w=w, counts=counts, offsets=offsets,
                row_token=row_token, row_of_slot=row_of_slot)


def rows_w4a8(tokens, x: np.ndarray, idx: np.ndarray, w: np.ndarray, expert,
              shared: Optional[tuple] = None, act: str = "silu", act_shared: str = "silu") -> np.ndarray:
    """W4A8 y for selected tokens given the routing; every quantisation is
    local to a row, so tokens can be evaluated one by one."""
    tokens = list(tokens)
    xd = mx_round_trip(np.asarray(x, np.float64)[tokens], "e4m3")
    k = idx.shape[1]
    y = np.zeros((len(tokens), xd.shape[1]))
    by_e = {}
    for n, t in enumerate(tokens):
        for j in range(k):
            by_e.setdefault(int(idx[t, j]), []).append((n, t, j))
    for e in sorted(by_e):
        items = by_e[e]
        w13, _, w2, _ = expert(e)
        o = expert_ffn_w4a8(xd[[n for n, _, _ in items]], w13, w2, act)
        for (n, t, j), orow in zip(items, o):
            y[n] += float(w[t, j]) * orow
    if shared is not None:
        y += expert_ffn_w4a8(xd, shared[0], shared[2], act_shared)
    return y
