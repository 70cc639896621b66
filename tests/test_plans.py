"""Which kernel shapes the layer plans, through moe_layer_plan (host planning
only, no GPU needed).

1. The full-size workloads take the shapes their measurements chose; a change
   of a threshold or a shape rule shows up here by name.
2. Together, the configurations the GPU parity tests run reach every shape of
   moe_plan_shape_t in each product that can take it, so no kernel shape the
   layer can launch goes untested on the GPU.
"""
import pytest

from gpu_helpers import problem
from sparse_mixture_experts_moe_amd import binding as B
from workloads import CONFIGS

import test_gpu_fused_combine as FC
import test_gpu_mx as MX
import test_gpu_parity as PAR
import test_gpu_w8a8 as W8
import test_gpu_w8a8_sub as WS


def plan(cfg, policy="auto", act_quant=0):
    return B.moe_layer_plan(problem(cfg, policy, act_quant=act_quant))


# (workload, act_quant) -> router, router K slices, gate/up, down, one-launch permutation
FULL = {
    ("qwen_decode", 0): ("stream64", 16, "tiled32x128", "tiled32x64", True),
    ("qwen_prefill", 0): ("tiled256x256", 4, "tiled256x256", "tiled128x512", False),
    ("gemma", 0): ("tiled128x256", 11, "tiled256x256", "tiled128x256", False),
    ("ling_prefill", 0): ("tiled256x256", 4, "tiled128x512", "tiled128x512", False),
    ("ling_decode", 0): ("tiled128x256", 32, "tiled32x128", "tiled32x128", True),
    ("ling_prefill", B.MOE_ACT_QUANT_FP8_ROW): ("tiled256x256", 4, "tiled128x512", "tiled128x512", False),
    ("ling_decode", B.MOE_ACT_QUANT_FP8_ROW): ("tiled128x256", 32, "tiled64x256", "tiled64x256", True),
    ("ling_prefill", B.MOE_ACT_QUANT_FP8_SUB): ("tiled256x256", 4, "tiled256x256", "tiled256x256", False),
    ("ling_decode", B.MOE_ACT_QUANT_FP8_SUB): ("tiled128x256", 32, "tiled64x256", "tiled64x256", True),
    ("ling_prefill_mxfp4", B.MOE_ACT_QUANT_MXFP8): ("tiled256x256", 4, "tiled128x512", "tiled128x512", False),
    ("ling_decode_mxfp4", B.MOE_ACT_QUANT_MXFP8): ("tiled128x256", 32, "tiled64x256", "tiled64x256", True),
}


@pytest.mark.parametrize("key", list(FULL), ids=lambda k: f"{k[0]}-aq{k[1]}")
def test_full_size_plans(key):
    name, aq = key
    got = plan(CONFIGS[name], act_quant=aq)
    want = dict(zip(("router", "router_slices", "gate_up", "down", "one_launch_permute"), FULL[key]))
    assert got == want, f"{name} act_quant={aq}: {got}"


def test_fp32_layer_streams_and_forced_policies():
    tiny = CONFIGS["tiny_fp32"]
    assert plan(tiny)["gate_up"].startswith("stream")
    cfg = CONFIGS["qwen_prefill"]
    assert plan(cfg, "stream")["gate_up"].startswith("stream")
    assert plan(cfg, "lds")["gate_up"] == "tiled256x256"


def _gpu_test_plans():
    """Plans of the layer configurations the GPU parity tests run."""
    out = []
    for cfg in PAR.SMALL.values():
        for pol in ("stream", "lds", "auto"):
            out.append(plan(cfg, pol))
    out += [plan(PAR.edge_config(over)) for over in PAR.EDGE]
    out += [plan(PAR.router_tall_config(D, E)) for D, E in PAR.ROUTER_TALL]
    for name in PAR.FULL:
        out.append(plan(CONFIGS[name]))
    out += [plan(c, act_quant=W8.AQ) for c in W8.SMALL.values()]
    out += [plan(c, act_quant=WS.AQ) for c in WS.SMALL.values()]
    out += [plan(c, act_quant=MX.AQ) for c in MX.SMALL.values()]
    out += [plan(c, act_quant=aq) for c, aq in FC.QUANT.values()]
    return out


def test_gpu_tests_reach_every_shape():
    plans = _gpu_test_plans()
    seen = {part: {p[part] for p in plans} for part in ("router", "gate_up", "down")}
    tiled_ffn = {"tiled256x256", "tiled128x512", "tiled128x256", "tiled32x128", "tiled64x256"}
    streams = {"stream16", "stream32", "stream64"}
    # the expert FFN's gated product: every streamed and every tiled shape
    assert streams | tiled_ffn <= seen["gate_up"], seen["gate_up"]
    # the down projection adds the 64-wide decode blocks
    assert streams | tiled_ffn | {"tiled32x64"} <= seen["down"], seen["down"]
    # the router: streamed (decode), 128-row and 256-row tiles (prefill)
    assert {"tiled128x256", "tiled256x256"} <= seen["router"] and seen["router"] & streams, seen["router"]
    assert any(p["one_launch_permute"] for p in plans) and not all(p["one_launch_permute"] for p in plans)
    assert any(p["router_slices"] > 1 for p in plans) and any(p["router_slices"] == 1 for p in plans)
