"""Dynamic per-token fp8 activation quantisation and the W8A8 layer.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline use this module; the HIP library never does, and the two share no code.

"Ling-2.6-1T with SGLang-JAX" page, section 5 (activation quantisation, and
per-channel direct_scaled_dot): the activations are quantised from bf16 to fp8
per token, dynamically, and the fp8 tokens and the fp8 per-channel weights go
into the matrix unit together; the float32 partial sums are scaled per token
and per channel only after the reduction.

What this module computes (the readings the page leaves open are marked):

  * quantize_rows: for each row a, s = max|a| / 448 in float32 (448 is the
    largest finite e4m3fn magnitude; reading: the dynamic scale maps the row's
    largest magnitude onto it; a row of zeros gets s = 1), then every element
    becomes the e4m3fn code nearest to a / s (float32 division), ties to the
    even code, magnitudes above 448 saturating to 448.  The encoder works from
    the format definition through the exact decode table of oracle.formats.
  * layer_w8a8: routing exactly as the plain layer (the router and the top-k
    softmax see the bf16 activations); the expert and shared FFNs run on the
    dequantised rows decode(q) * s; reading: the down projection's input h is
    quantised per row the same way, after being stored in bf16 as the GPU
    path stores it (the quantisation decision is taken in the precision of
    the stored value); everything else is float64.
  * the sub-channel variant ("Qwen 3.5 MoE on Ironwood" page, MoE track, the
    GMM v2 kernel: fp8 activations quantised per 512-element sub-channel):
    quantize_subchannel applies quantize_rows' rule to each run of `width`
    consecutive elements of a row (reading: the sub-channels are the
    consecutive 512-element slices of the reduction dimension, each with its
    own dynamic scale), so the dequantised row is decode(q[c]) * s[c // width];
    the W8A8 functions take width=None (one scale per row) or the slice width.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .formats import fp8_e4m3fn_table
from .moe import ACTS, permute, router_logits, topk_softmax

E4M3_MAX = 448.0

_TABLE = fp8_e4m3fn_table()
_POS_CODES = np.arange(0x7F)             # 0x00..0x7E: the finite non-negative codes
_POS_VALUES = _TABLE[_POS_CODES]         # strictly increasing, 0 .. 448


def encode_e4m3fn(v: np.ndarray) -> np.ndarray:
    """float32 values -> e4m3fn codes (uint8): nearest representable value,
    ties to the even code (even mantissa), saturating at +-448; the sign bit
    is the input's sign.  Non-finite inputs are outside the contract."""
    v = np.asarray(v, np.float32).astype(np.float64)
    mag = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.clip(np.searchsorted(_POS_VALUES, mag, side="left"), 0, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    return np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)


def quantize_rows(a: np.ndarray):
    """Rows of float32-representable values -> (codes uint8 [n,m], scales float32 [n])."""
    a32 = np.asarray(a, np.float64).astype(np.float32)
    amax = np.max(np.abs(a32), axis=1) if a32.shape[1] else np.zeros(a32.shape[0], np.float32)
    s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    return encode_e4m3fn(a32 / s[:, None]), s


def dequantize_rows(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    return _TABLE[np.asarray(q, np.uint8)] * np.asarray(s, np.float64)[:, None]


def quantize_subchannel(a: np.ndarray, width: int = 512):
    """Rows whose length is a multiple of width -> (codes uint8 [n,m], scales
    float32 [n, m // width]): quantize_rows on every width-element slice."""
    a32 = np.asarray(a, np.float64).astype(np.float32)
    n, m = a32.shape
    if m % width:
        raise ValueError("row length is not a multiple of the slice width")
    q, s = quantize_rows(a32.reshape(n * (m // width), width))
    return q.reshape(n, m), s.reshape(n, m // width)


def dequantize_subchannel(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    q = np.asarray(q, np.uint8)
    s = np.asarray(s, np.float64)
    width = q.shape[1] // s.shape[1]
    return _TABLE[q] * np.repeat(s, width, axis=1)


def quantize_dequantize(a: np.ndarray, width: Optional[int] = None) -> np.ndarray:
    """The dequantised rows decode(q) * s, one scale per row (width None) or
    per width-element slice."""
    if width is None:
        return dequantize_rows(*quantize_rows(a))
    return dequantize_subchannel(*quantize_subchannel(a, width))


def round_bf16(a: np.ndarray) -> np.ndarray:
    """float64 -> float32 -> bf16 (round to nearest even), back to float64."""
    b = np.asarray(a, np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def expert_ffn_w8a8(Xd: np.ndarray, w13: np.ndarray, s13: Optional[np.ndarray],
                    w2: np.ndarray, s2: Optional[np.ndarray], act: str,
                    width: Optional[int] = None) -> np.ndarray:
    """One gated expert on dequantised rows Xd: h is stored (bf16) and
    quantised (per row, or per width-element slice) before the down projection."""
    I = w13.shape[0] // 2
    gu = Xd @ w13.T
    if s13 is not None:
        gu = gu * np.asarray(s13, np.float64)[None, :]
    h = round_bf16(ACTS[act](gu[:, :I]) * gu[:, I:])
    hd = quantize_dequantize(h, width)
    o = hd @ w2.T
    if s2 is not None:
        o = o * np.asarray(s2, np.float64)[None, :]
    return o


def layer_w8a8(x: np.ndarray, wr: np.ndarray, k: int, expert, shared: Optional[tuple] = None,
               act: str = "silu", act_shared: str = "silu",
               logits_in: Optional[np.ndarray] = None, renormalize: bool = True,
               width: Optional[int] = None) -> dict:
    """The layer with dynamic fp8 activations (see the module text): one
    scale per token row (width None) or per width-element slice of it.
    x holds the bf16 activations as float64; expert / shared as for the plain
    layer.  Returns y and the routing artefacts."""
    x = np.asarray(x, np.float64)
    T, D = x.shape
    E = wr.shape[0]
    logits = router_logits(x, wr) if logits_in is None else np.asarray(logits_in, np.float32)
    idx, w = topk_softmax(logits, k, renormalize)
    counts, offsets, row_token, row_of_slot = permute(idx, E)
    if width is None:
        qx, sx = quantize_rows(x)
        xd = dequantize_rows(qx, sx)
    else:
        qx, sx = quantize_subchannel(x, width)
        xd = dequantize_subchannel(qx, sx)

    o_perm = np.zeros((T * k, D), dtype=np.float64)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        w13, s13, w2, s2 = expert(e)
        o_perm[r0:r1] = expert_ffn_w8a8(xd[row_token[r0:r1]], w13, s13, w2, s2, act, width)

    y = np.zeros((T, D), dtype=np.float64)
    for j in range(k):
        y += w[:, j].astype(np.float64)[:, None] * o_perm[row_of_slot.reshape(T, k)[:, j]]
    if shared is not None:
        w13s, s13s, w2s, s2s = shared
        y += expert_ffn_w8a8(xd, w13s, s13s, w2s, s2s, act_shared, width)
    return dict(y=y, logits=logits, idx=idx, w=w, counts=counts, offsets=offsets,
                row_token=row_token, row_of_slot=row_of_slot, x_codes=qx, x_scales=sx)


def rows_w8a8(tokens, x: np.ndarray, idx: np.ndarray, w: np.ndarray, expert,
              shared: Optional[tuple] = None, act: str = "silu", act_shared: str = "silu",
              width: Optional[int] = None) -> np.ndarray:
    """W8A8 y for the selected tokens, given the routing (idx, w rows for all
    tokens).  Every quantisation is within a row, so a token's output depends
    on its own row only and can be evaluated token by token, one expert at a time."""
    tokens = list(tokens)
    x = np.asarray(x, np.float64)
    xd = quantize_dequantize(x[tokens], width)
    k = idx.shape[1]
    y = np.zeros((len(tokens), x.shape[1]))
    by_e = {}
    for n, t in enumerate(tokens):
        for j in range(k):
            by_e.setdefault(int(idx[t, j]), []).append((n, t, j))
    for e in sorted(by_e):
        items = by_e[e]
        w13, s13, w2, s2 = expert(e)
        o = expert_ffn_w8a8(xd[[n for n, _, _ in items]], w13, s13, w2, s2, act, width)
        for (n, t, j), orow in zip(items, o):
            y[n] += float(w[t, j]) * orow
    if shared is not None:
        y += expert_ffn_w8a8(xd, *shared, act_shared, width)
    return y
