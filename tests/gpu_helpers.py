"""Helpers shared by the GPU parity tests (not collected by pytest).

The HIP side is reached only through the C ABI binding; the expected values come
only from `oracle/` on inputs drawn by `workloads/`.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle.formats import decode
from oracle.mx import decode_weight
from oracle.moe import (expert_ffn, experts_from_bits, layer, permute, rel_err,
                        shared_from_bits, topk_softmax)
from sparse_mixture_experts_moe_amd import binding as B
from workloads import host_expert, host_shared, to_bits

TOL = {"f32": 1e-4, "bf16": 1e-2, "fp8": 3e-2}


def tol_for(cfg) -> float:
    return TOL[cfg.w_dtype] if cfg.w_dtype == "fp8" else TOL[cfg.act_dtype]


def problem(cfg, policy="auto", renormalize=True, act_quant=0) -> B.MoeProblem:
    return B.make_problem(cfg.T, cfg.D, cfg.E, cfg.k, cfg.I, cfg.I_shared, cfg.act, cfg.act_shared,
                          cfg.act_dtype, cfg.w_dtype, cfg.shared_w_dtype, policy, renormalize,
                          act_quant)


def to_device(wl, dev="cuda"):
    """Move every tensor of a workload to the GPU (in place) and return it."""
    for n in ("x", "wr", "w13", "w2", "s13", "s2", "w13s", "w2s", "s13s", "s2s"):
        t = getattr(wl, n)
        if t is not None:
            setattr(wl, n, t.to(dev))
    return wl


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 value of a GPU/CPU tensor of f32 / bf16 storage."""
    dt = {torch.float32: "f32", torch.bfloat16: "bf16"}[t.dtype]
    return decode(to_bits(t), dt)


def run_layer(wl, policy="auto", logits_in=None, want=("logits_out", "topk_idx_out", "topk_w_out",
                                                       "counts_out", "offsets_out",
                                                       "row_token_out", "row_of_slot_out"),
              renormalize=True, act_quant=0):
    p = problem(wl.cfg, policy, renormalize, act_quant)
    res = B.run_layer(p, wl.x, wl.w13, wl.w2, w_router=wl.wr, s13=wl.s13, s2=wl.s2,
                      w13_shared=wl.w13s, s13_shared=wl.s13s, w2_shared=wl.w2s, s2_shared=wl.s2s,
                      logits_in=logits_in, want=want)
    torch.cuda.synchronize()
    return res


def oracle_inputs(wl):
    """Decoded x, Wr and expert/shared accessors (experts fetched one by one)."""
    c = wl.cfg
    x = decode(to_bits(wl.x), c.act_dtype)
    wr = decode(to_bits(wl.wr), c.act_dtype)

    def expert(e):
        w13, s13, w2, s2 = host_expert(wl, e)
        a, sa = decode_weight(w13, s13, c.w_dtype)
        b, sb = decode_weight(w2, s2, c.w_dtype)
        return a, sa, b, sb
    sh = host_shared(wl)
    shared = None
    if sh is not None:
        a, sa = decode_weight(sh[0], sh[1], c.shared_w_dtype)
        b, sb = decode_weight(sh[2], sh[3], c.shared_w_dtype)
        shared = (a, sa, b, sb)
    return x, wr, expert, shared


def oracle_layer(wl, logits_in=None, keep=False, renormalize=True):
    x, wr, expert, shared = oracle_inputs(wl)
    c = wl.cfg
    return layer(x, wr, c.k, expert, shared, c.act, c.act_shared, logits_in=logits_in, keep=keep,
                 renormalize=renormalize)


def oracle_rows(wl, tokens, idx, w):
    """y for selected tokens from their routing, one decoded expert at a time."""
    x, _, expert, shared = oracle_inputs(wl)
    c = wl.cfg
    tokens = list(tokens)
    y = np.zeros((len(tokens), c.D))
    by_e = {}
    for n, t in enumerate(tokens):
        for j in range(c.k):
            by_e.setdefault(int(idx[t, j]), []).append((n, t, j))
    for e, items in by_e.items():
        w13, s13, w2, s2 = expert(e)
        X = x[[t for _, t, _ in items]]
        o = expert_ffn(X, w13, s13, w2, s2, c.act)
        for (n, t, j), orow in zip(items, o):
            y[n] += float(w[t, j]) * orow
    if shared is not None:
        y += expert_ffn(x[tokens], *shared, c.act_shared)
    return y


def oracle_routing_from_logits(logits_ref, k, E):
    idx, w = topk_softmax(logits_ref, k)
    counts, offsets, row_token, row_of_slot = permute(idx, E)
    return dict(idx=idx, w=w, counts=counts, offsets=offsets, row_token=row_token,
                row_of_slot=row_of_slot)


__all__ = ["TOL", "tol_for", "problem", "to_device", "f64", "run_layer", "oracle_layer",
           "oracle_rows", "oracle_inputs", "oracle_routing_from_logits", "rel_err",
           "experts_from_bits", "shared_from_bits"]
