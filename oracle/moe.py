"""Plain float64 CPU oracle of the routed MoE FFN layer.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline use this module; the HIP library never does, and the two share no code.

What it computes, step by step, in float64 with no blocking or fusion:

  y = Router(x) + SharedExpert(x)
      -- "Qwen 3.5 MoE on Ironwood" page, model-architecture section (the MoE
         FFN equation with the always-executed shared expert).

  1. logits l = x . Wr^T, evaluated in float64 and rounded once to float32
     (the gate is fed fp32 values: "CANN Qwen3-MoE" page, RMSNorm fusion
     section, where the norm emits fp32 for the gate).
  2. top-k softmax with renormalisation: take the k largest float32 logits in
     descending order, equal values going to the lower expert index, and weight
     them w_j = exp(l_j - l_0) / sum_m exp(l_m - l_0).  This equals softmax over
     all experts, then top-k, then renormalising the k probabilities ("Qwen 3.5
     MoE on Ironwood", model architecture), and equals the fused top-k-softmax
     op ("CANN Qwen3-MoE", GMM enablement and routing optimisation), because the
     full-softmax denominator cancels.  Without renormalisation (the router as
     a linear layer plus softmax, "TP MoE" page, section 3.3) the weights are
     the selected experts' softmax probabilities over all experts.
  3. permutation ("init routing" / "compute expert tokens" on the CANN
     Qwen3-MoE page): per-expert counts, their exclusive prefix sum, and the
     stable order of the flattened (token, slot) assignments by expert id, which
     inside an expert is ascending token order.
  4. per expert e over its rows X_e: [g | u] = X_e . W13[e]^T (times the
     per-output-channel scale after the reduction, "Ling-2.6-1T with SGLang-JAX"
     page, section 5, per-channel direct_scaled_dot), h = act(g) * u with
     SwiGLU act = SiLU on the first half of the chunked projection ("CANN
     Qwen3-MoE", MoE TP compute decomposition) or GEGLU act = tanh-GELU ("Gemma-4
     model optimisation report", section 2), then o = h . W2[e]^T (times s2).
  5. the shared expert / dense MLP: the same FFN on every token, weight 1.
  6. combine ("finalize routing" on the CANN Qwen3-MoE page): y[t] =
     sum_j w[t,j] * o[row of slot (t,j)] + shared[t].
"""
from __future__ import annotations

from typing import Callable, Optional

import numpy as np

from .formats import decode

ExpertFn = Callable[[int], tuple]


# ---------------------------------------------------------------- activations
def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z / (1 + exp(-z))."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def gelu_tanh(z: np.ndarray) -> np.ndarray:
    """tanh-approximated GELU: 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3)))."""
    return 0.5 * z * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (z + 0.044715 * z ** 3)))


ACTS = {"silu": silu, "gelu_tanh": gelu_tanh}


# ---------------------------------------------------------------- step 1
def router_logits(x: np.ndarray, wr: np.ndarray) -> np.ndarray:
    """x [T,D] f64, wr [E,D] f64 -> float32 logits [T,E] (one rounding)."""
    return (np.asarray(x, np.float64) @ np.asarray(wr, np.float64).T).astype(np.float32)


# ---------------------------------------------------------------- step 2
def topk_softmax(logits: np.ndarray, k: int, renormalize: bool = True):
    """float32 logits [T,E] -> (idx int32 [T,k], w float32 [T,k]).

    renormalize=False keeps the selected experts' plain softmax probabilities
    over all E experts, w_j = exp(l_j - l_0) / sum_e exp(l_e - l_0) (softmax
    gating without renormalisation: the router is a linear layer followed by a
    softmax, "TP MoE" page, section 3.3).
    """
    l32 = np.asarray(logits, dtype=np.float32)
    T, E = l32.shape
    if not 1 <= k <= E:
        raise ValueError("k out of range")
    # a stable sort of the negated values keeps equal values in index order;
    # -0.0 and +0.0 compare equal, so they tie as well.
    order = np.argsort(-l32, axis=1, kind="stable")[:, :k]
    idx = order.astype(np.int32)
    top = np.take_along_axis(l32, order, axis=1).astype(np.float64)
    ex = np.exp(top - top[:, :1])
    if renormalize:
        den = ex.sum(axis=1, keepdims=True)
    else:
        den = np.exp(l32.astype(np.float64) - top[:, :1]).sum(axis=1, keepdims=True)
    w = ex / den
    return idx, w.astype(np.float32)


# ---------------------------------------------------------------- step 3
def permute(idx: np.ndarray, E: int):
    """topk idx [T,k] -> counts [E], offsets [E+1], row_token [T*k], row_of_slot [T*k]."""
    idx = np.asarray(idx)
    T, k = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    order = np.argsort(flat, kind="stable")          # sorted row r -> slot a
    row_token = order // k
    row_of_slot = np.empty(T * k, dtype=np.int64)
    row_of_slot[order] = np.arange(T * k)
    return (counts.astype(np.int32), offsets.astype(np.int32),
            row_token.astype(np.int32), row_of_slot.astype(np.int32))


# ---------------------------------------------------------------- steps 4/5
def expert_ffn(X: np.ndarray, w13: np.ndarray, s13: Optional[np.ndarray],
               w2: np.ndarray, s2: Optional[np.ndarray], act: str,
               return_h: bool = False):
    """One gated expert on the rows X [n,D] (float64 throughout).

    w13 [2I,D]: rows [0,I) gate, rows [I,2I) up; w2 [D,I]; s13 [2I], s2 [D]
    are per-output-channel scales applied after the reduction (None = 1).
    """
    I = w13.shape[0] // 2
    gu = X @ w13.T
    if s13 is not None:
        gu = gu * np.asarray(s13, np.float64)[None, :]
    h = ACTS[act](gu[:, :I]) * gu[:, I:]
    o = h @ w2.T
    if s2 is not None:
        o = o * np.asarray(s2, np.float64)[None, :]
    return (o, h) if return_h else o


def experts_from_bits(w13_bits, s13, w2_bits, s2, dtype: str) -> ExpertFn:
    """Accessor e -> decoded (w13, s13, w2, s2) over raw [E,...] storage (for
    MXFP4 the block scales are folded into the decoded weights and s = None)."""
    from .mx import decode_weight

    def get(e):
        w13, a = decode_weight(w13_bits[e], None if s13 is None else s13[e], dtype)
        w2, b = decode_weight(w2_bits[e], None if s2 is None else s2[e], dtype)
        return w13, a, w2, b
    return get


def shared_from_bits(w13_bits, s13, w2_bits, s2, dtype: str):
    from .mx import decode_weight
    w13, a = decode_weight(w13_bits, s13, dtype)
    w2, b = decode_weight(w2_bits, s2, dtype)
    return w13, a, w2, b


# ---------------------------------------------------------------- whole layer
def layer(x: np.ndarray, wr: np.ndarray, k: int, expert: ExpertFn,
          shared: Optional[tuple] = None, act: str = "silu",
          act_shared: str = "silu", logits_in: Optional[np.ndarray] = None,
          keep: bool = False, renormalize: bool = True) -> dict:
    """The full layer on decoded float64 inputs.

    x [T,D], wr [E,D]; expert(e) -> (w13, s13, w2, s2) decoded; shared is the
    decoded (w13s, s13s, w2s, s2s) tuple or None.  With `logits_in` the router
    product is skipped and the given float32 logits are routed;
    renormalize=False gives the plain softmax weights (see topk_softmax).
    Returns y (float64) and every routing artefact; with keep=True also the
    per-row h and o (float64, sorted-row order) and the shared output.
    """
    x = np.asarray(x, np.float64)
    T, D = x.shape
    E = wr.shape[0]
    logits = router_logits(x, wr) if logits_in is None else np.asarray(logits_in, np.float32)
    idx, w = topk_softmax(logits, k, renormalize)
    counts, offsets, row_token, row_of_slot = permute(idx, E)

    o_perm = np.zeros((T * k, D), dtype=np.float64)
    h_rows = [] if keep else None
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        w13, s13, w2, s2 = expert(e)
        res = expert_ffn(x[row_token[r0:r1]], w13, s13, w2, s2, act, return_h=keep)
        if keep:
            o_perm[r0:r1], h = res
            h_rows.append((r0, h))
        else:
            o_perm[r0:r1] = res

    y = np.zeros((T, D), dtype=np.float64)
    for j in range(k):
        y += w[:, j].astype(np.float64)[:, None] * o_perm[row_of_slot.reshape(T, k)[:, j]]
    s_out = None
    if shared is not None:
        w13s, s13s, w2s, s2s = shared
        s_out = expert_ffn(x, w13s, s13s, w2s, s2s, act_shared)
        y += s_out

    out = dict(y=y, logits=logits, idx=idx, w=w, counts=counts, offsets=offsets,
               row_token=row_token, row_of_slot=row_of_slot)
    if keep:
        I = h_rows[0][1].shape[1] if h_rows else 0
        h_perm = np.zeros((T * k, I), dtype=np.float64)
        for r0, h in h_rows:
            h_perm[r0:r0 + h.shape[0]] = h
        out.update(o_perm=o_perm, h_perm=h_perm, shared_out=s_out)
    return out


def layer_tokens(tokens, x: np.ndarray, idx: np.ndarray, w: np.ndarray,
                 expert: ExpertFn, shared: Optional[tuple] = None,
                 act: str = "silu", act_shared: str = "silu") -> np.ndarray:
    """y for a subset of tokens, given their routing (idx, w rows for all T).

    Evaluates step 6 from the definition for the selected tokens only: every
    (token, slot) assignment's expert FFN on that token's row, weighted and
    summed, plus the shared branch.  Experts are visited in ascending id, each
    once, over all selected rows routed to it, so one decoded expert is held at
    a time.
    """
    x = np.asarray(x, np.float64)
    tokens = list(tokens)
    y = np.zeros((len(tokens), x.shape[1]), dtype=np.float64)
    by_e = {}
    for n, t in enumerate(tokens):
        for j in range(idx.shape[1]):
            by_e.setdefault(int(idx[t, j]), []).append((n, t, j))
    for e in sorted(by_e):
        items = by_e[e]
        w13, s13, w2, s2 = expert(e)
        o = expert_ffn(x[[t for _, t, _ in items]], w13, s13, w2, s2, act)
        for (n, t, j), orow in zip(items, o):
            y[n] += float(w[t, j]) * orow
    if shared is not None:
        w13s, s13s, w2s, s2s = shared
        y += expert_ffn(x[tokens], w13s, s13s, w2s, s2s, act_shared)
    return y


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref| over the whole tensor, in float64."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(got - ref)) if ref.size else 0.0
    return float(num / den) if den > 0 else float(num)
