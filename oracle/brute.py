"""Brute-force per-token dense evaluation of the MoE layer (tiny inputs only).

Test infrastructure, like the rest of `oracle/`.  It shares the definition of
the layer with `oracle.moe` but none of its structure: no permutation, no
per-expert batching, and the routing weights are formed the way the "Qwen 3.5
MoE on Ironwood" page states them (softmax over every expert, select the top
10 -- here top k -- then renormalise the selected probabilities), with the
selection done by Python's own sort of (-logit, expert) keys.
"""
from __future__ import annotations

import math

import numpy as np


def _act(name: str, z: float) -> float:
    if name == "silu":
        # z * sigmoid(z), written with the sign split so exp never overflows
        if z >= 0:
            return z / (1.0 + math.exp(-z))
        ez = math.exp(z)
        return z * ez / (1.0 + ez)
    if name == "gelu_tanh":
        c = math.sqrt(2.0 / math.pi)
        return 0.5 * z * (1.0 + math.tanh(c * (z + 0.044715 * z * z * z)))
    raise ValueError(name)


def _ffn_token(xt, w13, s13, w2, s2, act):
    """One token through one gated expert, matrix-vector products only."""
    I = w13.shape[0] // 2
    gu = w13 @ xt
    if s13 is not None:
        gu = gu * s13
    h = np.array([_act(act, float(gu[i])) * float(gu[I + i]) for i in range(I)])
    o = w2 @ h
    if s2 is not None:
        o = o * s2
    return o


def brute_force_layer(x, wr, k, experts, shared=None, act="silu",
                      act_shared="silu"):
    """x [T,D] f64; wr [E,D] f64; experts: list of decoded (w13,s13,w2,s2).

    Returns (y [T,D] f64, selected [T][k] lists, gates [T,E] f64).
    """
    T, D = x.shape
    E = wr.shape[0]
    y = np.zeros((T, D))
    gates = np.zeros((T, E))
    chosen_all = []
    for t in range(T):
        logit = [np.float32(np.dot(x[t], wr[e])) for e in range(E)]
        lf = [float(v) for v in logit]
        m = max(lf)
        p = [math.exp(v - m) for v in lf]
        z = sum(p)
        p = [v / z for v in p]                               # softmax over all E
        chosen = sorted(range(E), key=lambda e: (-lf[e], e))[:k]
        ps = sum(p[e] for e in chosen)
        for e in chosen:
            gates[t, e] = p[e] / ps                          # renormalised
            y[t] += gates[t, e] * _ffn_token(x[t], *experts[e], act)
        if shared is not None:
            y[t] += _ffn_token(x[t], *shared, act_shared)
        chosen_all.append(chosen)
    return y, chosen_all, gates
