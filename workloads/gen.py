"""Layer configurations and the seeded input recipe.

The six layer shapes are the ones the pages describe:
  * a tiny fp32 layer (parity only);
  * the Qwen3.5-397B MoE layer (512 experts, intermediate 1024, top-10 softmax,
    one always-on shared expert) as a 64-token decode step and an 8192-token
    prefill -- "Qwen 3.5 MoE on Ironwood" page, model-architecture section;
  * the Gemma-4-26B-A4B layer (128 experts, top-8, GEGLU intermediate 704,
    summed with a parallel dense MLP of intermediate 2112) -- "Gemma-4 model
    optimisation report" page, section 2 (model structure);
  * the Ling-2.6-1T layer (hidden 8192, 256 experts, top-8, one shared expert,
    per-channel fp8 expert weights) at 16384-token prefill and 512-token decode
    -- "Ling-2.6-1T with SGLang-JAX" page, section 1 (cost model).

Recipe (both sides read the same tensors):
  * x and the router weight are drawn in fp32 from a CPU torch.Generator seeded
    `seed`, in that order: x ~ N(0,1) [T,D], Wr ~ N(0,1/D) [E,D];
  * for the Zipf-skewed prefill, a second CPU generator seeded `seed+1` draws a
    permutation that gives each expert a rank rho_e in 1..E and row e of Wr is
    scaled by rho_e**-ZIPF_ALPHA;
  * expert weights come from a generator seeded `seed+2` on `weight_device`,
    expert by expert: W13[e] ~ N(0,1/D) [2I,D], then W2[e] ~ N(0,1/I) [D,I];
    then the shared/dense branch W13s [2Is,D], W2s [D,Is];
  * casts: bf16 by round-to-nearest-even; fp8 e4m3fn per output row with
    s[n] = amax_n/448 and q = RNE(clamp(W[n,:]/s[n], -448, 448)); MXFP4 (the
    W4A8 weights of the CANN Qwen3-MoE page, in the Open Compute Project
    microscaling format): per block of 32 consecutive K elements the E8M0 scale
    exponent is floor(log2 amax) - 2, the e2m1 codes are the nearest values of
    W / 2**exp (ties to the even code, saturating at 6).  MXFP4 storage: two
    codes per byte (element 2j in the low nibble), [.., N, K/2]; scales grouped
    by 128 K elements, [.., K/128, N, 4] (a row's four block scales of a group
    side by side).
Rows [0,I) of W13 are the gate projection, rows [I,2I) the up projection.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

# Exponent of the per-expert router gains rho**-alpha used for the Zipf-skewed
# prefill.  Fitted by tests/golden/fit_zipf_alpha.py so that the least-squares
# slope of log(per-expert load) against log(load rank) is -1 for seed 0.
ZIPF_ALPHA = 0.2234


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int          # tokens
    D: int          # hidden size
    E: int          # routed experts
    k: int          # experts per token
    I: int          # routed expert intermediate size
    I_shared: int   # shared expert / dense MLP intermediate size (0 = none)
    act: str        # "silu" (SwiGLU) or "gelu_tanh" (GEGLU)
    act_shared: str
    act_dtype: str  # "f32" | "bf16"  (x, router weight, y)
    w_dtype: str    # "f32" | "bf16" | "fp8" | "mxfp4"  (routed W13 / W2)
    shared_w_dtype: str
    zipf: bool = False

    @property
    def rows(self) -> int:
        return self.T * self.k


def _cfg(name, T, D, E, k, I, I_shared, act, act_dtype, w_dtype, zipf=False):
    return MoEConfig(name, T, D, E, k, I, I_shared, act, act, act_dtype, w_dtype,
                     w_dtype, zipf)


CONFIGS = {
    "tiny_fp32": _cfg("tiny_fp32", 64, 256, 8, 2, 128, 0, "silu", "f32", "f32"),
    "qwen_decode": _cfg("qwen_decode", 64, 4096, 512, 10, 1024, 1024, "silu", "bf16", "bf16"),
    "qwen_prefill": _cfg("qwen_prefill", 8192, 4096, 512, 10, 1024, 1024, "silu", "bf16", "bf16",
                         zipf=True),
    "gemma": _cfg("gemma", 2048, 2816, 128, 8, 704, 2112, "gelu_tanh", "bf16", "bf16"),
    "ling_prefill": _cfg("ling_prefill", 16384, 8192, 256, 8, 2048, 2048, "silu", "bf16", "fp8"),
    "ling_decode": _cfg("ling_decode", 512, 8192, 256, 8, 2048, 2048, "silu", "bf16", "fp8"),
    # the Ling layer with MXFP4 expert weights (the W4A8 setting of the CANN
    # Qwen3-MoE page); not one of the five configurations the pages measure
    "ling_prefill_mxfp4": _cfg("ling_prefill_mxfp4", 16384, 8192, 256, 8, 2048, 2048, "silu", "bf16",
                               "mxfp4"),
    "ling_decode_mxfp4": _cfg("ling_decode_mxfp4", 512, 8192, 256, 8, 2048, 2048, "silu", "bf16",
                              "mxfp4"),
}


def shrink(cfg: MoEConfig, **over) -> MoEConfig:
    """A copy of `cfg` with some fields replaced (smaller shapes for tests)."""
    d = dataclasses.asdict(cfg)
    d.update(over)
    if "name" not in over:
        d["name"] = cfg.name + "_small"
    return MoEConfig(**d)


_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclasses.dataclass
class Workload:
    cfg: MoEConfig
    seed: int
    x: torch.Tensor                 # [T,D] act dtype
    wr: torch.Tensor                # [E,D] act dtype
    w13: torch.Tensor               # [E,2I,D] f32 | bf16 | float8_e4m3fn
    w2: torch.Tensor                # [E,D,I]
    s13: Optional[torch.Tensor]     # [E,2I] f32 (fp8 only)
    s2: Optional[torch.Tensor]      # [E,D] f32 (fp8 only)
    w13s: Optional[torch.Tensor]    # [2Is,D]
    w2s: Optional[torch.Tensor]     # [D,Is]
    s13s: Optional[torch.Tensor]    # [2Is]
    s2s: Optional[torch.Tensor]     # [D]


def _quant_fp8_rows(w: torch.Tensor):
    """Per-output-row fp8 e4m3fn quantisation of an fp32 matrix [..., N, K]."""
    amax = w.abs().amax(dim=-1)
    s = amax / 448.0
    s = torch.where(s > 0, s, torch.ones_like(s))
    q = (w / s.unsqueeze(-1)).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q, s.to(torch.float32)


_E2M1_MAG = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def _quant_mxfp4(w: torch.Tensor):
    """MXFP4 quantisation of an fp32 matrix [N, K] (K a multiple of 128):
    (packed codes uint8 [N, K/2], scales uint8 [K/128, N, 4])."""
    N, K = w.shape
    blocks = w.reshape(N, K // 32, 32)
    amax = blocks.abs().amax(dim=2)
    _, ex = torch.frexp(amax)                            # amax = m * 2**ex, m in [0.5, 1)
    shared = torch.where(amax > 0, ex - 1, torch.full_like(ex, -127)) - 2
    shared = shared.clamp(-127, 127)
    scaled = blocks / torch.exp2(shared.to(torch.float32)).unsqueeze(-1)
    mag = scaled.abs().clamp(max=6.0)
    vals = torch.tensor(_E2M1_MAG, device=w.device)
    mids = (vals[1:] + vals[:-1]) / 2
    idx = torch.bucketize(mag, mids, right=True)         # a tie goes to the upper code here
    tie = (idx > 0) & (mag == mids[(idx - 1).clamp(min=0)])
    idx = torch.where(tie & (idx % 2 == 1), idx - 1, idx)   # ... and back to the even one
    codes = (idx | torch.where(torch.signbit(scaled), 8, 0)).to(torch.uint8).reshape(N, K)
    packed = codes[:, 0::2] | (codes[:, 1::2] << 4)
    scales = (shared + 127).to(torch.uint8).reshape(N, K // 128, 4).permute(1, 0, 2).contiguous()
    return packed, scales


def _cast(w: torch.Tensor, dtype: str):
    if dtype == "fp8":
        return _quant_fp8_rows(w)
    if dtype == "mxfp4":
        return _quant_mxfp4(w)
    return w.to(_TORCH_DT[dtype]), None


def router_inputs(cfg: MoEConfig, seed: int = 0, zipf_alpha: Optional[float] = None):
    """x [T,D] and the router weight [E,D], already cast to the activation dtype."""
    T, D, E = cfg.T, cfg.D, cfg.E
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn(T, D, generator=g, dtype=torch.float32)
    wr = torch.randn(E, D, generator=g, dtype=torch.float32) / math.sqrt(D)
    if cfg.zipf:
        alpha = ZIPF_ALPHA if zipf_alpha is None else zipf_alpha
        g1 = torch.Generator(device="cpu").manual_seed(seed + 1)
        rank = torch.randperm(E, generator=g1).to(torch.float64) + 1.0
        wr = wr * rank.pow(-alpha).to(torch.float32).unsqueeze(1)
    adt = _TORCH_DT[cfg.act_dtype]
    return x.to(adt), wr.to(adt)


def generate(cfg: MoEConfig, seed: int = 0, weight_device: str = "cpu",
             zipf_alpha: Optional[float] = None) -> Workload:
    D, E, I, Is = cfg.D, cfg.E, cfg.I, cfg.I_shared
    x, wr = router_inputs(cfg, seed, zipf_alpha)
    dev = torch.device(weight_device)
    gw = torch.Generator(device=dev).manual_seed(seed + 2)
    mx = cfg.w_dtype == "mxfp4"
    wdt = {"fp8": torch.float8_e4m3fn, "mxfp4": torch.uint8}.get(cfg.w_dtype, _TORCH_DT.get(cfg.w_dtype))
    w13 = torch.empty((E, 2 * I, D // 2 if mx else D), dtype=wdt, device=dev)
    w2 = torch.empty((E, D, I // 2 if mx else I), dtype=wdt, device=dev)
    fp8 = cfg.w_dtype == "fp8"
    s13 = s2 = None
    if fp8:
        s13 = torch.empty((E, 2 * I), dtype=torch.float32, device=dev)
        s2 = torch.empty((E, D), dtype=torch.float32, device=dev)
    if mx:
        s13 = torch.empty((E, D // 128, 2 * I, 4), dtype=torch.uint8, device=dev)
        s2 = torch.empty((E, I // 128, D, 4), dtype=torch.uint8, device=dev)
    for e in range(E):
        a = torch.randn((2 * I, D), generator=gw, device=dev) / math.sqrt(D)
        q, s = _cast(a, cfg.w_dtype)
        w13[e].copy_(q)
        if s is not None:
            s13[e].copy_(s)
        b = torch.randn((D, I), generator=gw, device=dev) / math.sqrt(I)
        q, s = _cast(b, cfg.w_dtype)
        w2[e].copy_(q)
        if s is not None:
            s2[e].copy_(s)
    w13s = w2s = s13s = s2s = None
    if Is:
        a = torch.randn((2 * Is, D), generator=gw, device=dev) / math.sqrt(D)
        w13s, s13s = _cast(a, cfg.shared_w_dtype)
        b = torch.randn((D, Is), generator=gw, device=dev) / math.sqrt(Is)
        w2s, s2s = _cast(b, cfg.shared_w_dtype)
    return Workload(cfg, seed, x, wr, w13, w2, s13, s2, w13s, w2s, s13s, s2s)


def to_bits(t: Optional[torch.Tensor]):
    """Raw storage of a tensor as a host numpy array: uint16 for bf16, uint8 for
    fp8 e4m3fn, float32 for fp32 (no value conversion happens here)."""
    if t is None:
        return None
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    if t.dtype in (torch.float32, torch.uint8):
        return t.numpy()
    raise TypeError(f"unsupported dtype {t.dtype}")


def host_expert(wl: Workload, e: int):
    """Raw host copies of expert e's weights: (w13, s13, w2, s2)."""
    s13 = None if wl.s13 is None else wl.s13[e].to("cpu").numpy()
    s2 = None if wl.s2 is None else wl.s2[e].to("cpu").numpy()
    return to_bits(wl.w13[e]), s13, to_bits(wl.w2[e]), s2


def host_shared(wl: Workload):
    """Raw host copies of the shared branch's weights, or None."""
    if wl.w13s is None:
        return None
    s13 = None if wl.s13s is None else wl.s13s.to("cpu").numpy()
    s2 = None if wl.s2s is None else wl.s2s.to("cpu").numpy()
    return to_bits(wl.w13s), s13, to_bits(wl.w2s), s2
