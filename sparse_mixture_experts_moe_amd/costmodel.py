"""Algorithmic FLOP and byte counts of the routed MoE FFN layer, and rooflines.

The counts are those of the method itself, not of padded or re-read work, in
the form the "Ling-2.6-1T with SGLang-JAX" page uses for its cost model
(section 1): a gated expert over n rows costs 2 matrices x 2*n*D*I FLOP for the
gate/up projection (FFN1) and 2*n*I*D for the down projection (FFN2); an
expert's weights are 3*D*I elements; a lower bound is work / peak rate.

MI355X peaks used for rooflines are the vendor's dense figures.
"""
from __future__ import annotations

DTYPE_BYTES = {"f32": 4, "bf16": 2, "fp8": 1, "mxfp4": 0.5}


def _scale_bytes(n_rows: int, K: int, w_dtype: str) -> float:
    """Scales of an [n_rows, K] weight: fp32 per row (fp8), one E8M0 byte per
    32 elements (MXFP4), none otherwise."""
    if w_dtype == "fp8":
        return 4.0 * n_rows
    if w_dtype == "mxfp4":
        return n_rows * K / 32.0
    return 0.0


# MI355X published dense peaks
PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "fp8": 5000.0, "f32": 157.3, "f64": 78.6}


def ffn1_flops(rows: int, D: int, I: int) -> float:
    """Gate + up projections of `rows` rows: 2 matrices x 2*rows*D*I."""
    return 2.0 * (2.0 * rows * D * I)


def ffn2_flops(rows: int, D: int, I: int) -> float:
    """Down projection: 2*rows*I*D."""
    return 2.0 * rows * I * D


def ffn_flops(rows: int, D: int, I: int) -> float:
    return ffn1_flops(rows, D, I) + ffn2_flops(rows, D, I)


def router_flops(T: int, D: int, E: int) -> float:
    return 2.0 * T * E * D


def expert_weight_bytes(D: int, I: int, w_dtype: str, with_scales: bool = False) -> float:
    """W13 (2I x D) + W2 (D x I) of one expert, plus their scales."""
    b = 3.0 * D * I * DTYPE_BYTES[w_dtype]
    if with_scales:
        b += _scale_bytes(2 * I, D, w_dtype) + _scale_bytes(D, I, w_dtype)
    return b


def w13_bytes(D: int, I: int, w_dtype: str) -> float:
    return 2.0 * I * D * DTYPE_BYTES[w_dtype] + _scale_bytes(2 * I, D, w_dtype)


def w2_bytes(D: int, I: int, w_dtype: str) -> float:
    return 1.0 * D * I * DTYPE_BYTES[w_dtype] + _scale_bytes(D, I, w_dtype)


def layer_flops(cfg) -> float:
    f = router_flops(cfg.T, cfg.D, cfg.E) + ffn_flops(cfg.T * cfg.k, cfg.D, cfg.I)
    if cfg.I_shared:
        f += ffn_flops(cfg.T, cfg.D, cfg.I_shared)
    return f


def gemm_flops(cfg) -> float:
    """Grouped-GEMM FLOP only (routed + shared), the MFMA-utilisation numerator."""
    f = ffn_flops(cfg.T * cfg.k, cfg.D, cfg.I)
    if cfg.I_shared:
        f += ffn_flops(cfg.T, cfg.D, cfg.I_shared)
    return f


def layer_bytes(cfg, touched_experts: int) -> float:
    """x + Wr + every touched expert's weights once (+scales) + shared + y."""
    a = DTYPE_BYTES[cfg.act_dtype]
    b = cfg.T * cfg.D * a + cfg.E * cfg.D * a
    b += touched_experts * expert_weight_bytes(cfg.D, cfg.I, cfg.w_dtype, True)
    if cfg.I_shared:
        b += expert_weight_bytes(cfg.D, cfg.I_shared, cfg.shared_w_dtype, True)
    b += cfg.T * cfg.D * a
    return b


def gemm1_bytes(cfg, touched_experts: int) -> float:
    """Algorithmic bytes of one fused gate/up launch (routed + shared groups):
    each touched expert's W13 (+scales) once, the x rows read once, h written."""
    a = DTYPE_BYTES[cfg.act_dtype]
    b = touched_experts * w13_bytes(cfg.D, cfg.I, cfg.w_dtype)
    b += cfg.T * cfg.D * a                              # x, every token once
    b += cfg.T * cfg.k * cfg.I * a                      # h of the routed rows
    if cfg.I_shared:
        b += w13_bytes(cfg.D, cfg.I_shared, cfg.shared_w_dtype)
        b += cfg.T * cfg.I_shared * a
    return b


def gemm2_bytes(cfg, touched_experts: int) -> float:
    """Algorithmic bytes of one down-projection launch: W2 once per touched
    expert, h read, o written (routed rows + shared rows)."""
    a = DTYPE_BYTES[cfg.act_dtype]
    b = touched_experts * w2_bytes(cfg.D, cfg.I, cfg.w_dtype)
    b += cfg.T * cfg.k * (cfg.I + cfg.D) * a
    if cfg.I_shared:
        b += w2_bytes(cfg.D, cfg.I_shared, cfg.shared_w_dtype)
        b += cfg.T * (cfg.I_shared + cfg.D) * a
    return b


def gemm1_flops(cfg) -> float:
    f = ffn1_flops(cfg.T * cfg.k, cfg.D, cfg.I)
    if cfg.I_shared:
        f += ffn1_flops(cfg.T, cfg.D, cfg.I_shared)
    return f


def gemm2_flops(cfg) -> float:
    f = ffn2_flops(cfg.T * cfg.k, cfg.D, cfg.I)
    if cfg.I_shared:
        f += ffn2_flops(cfg.T, cfg.D, cfg.I_shared)
    return f


def bound_ms(flops: float, nbytes: float, peak_tflops: float, peak_gbs: float = PEAK_HBM_GBS):
    """(compute-bound ms, memory-bound ms)."""
    return flops / (peak_tflops * 1e9), nbytes / (peak_gbs * 1e6)
