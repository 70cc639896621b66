"""The fused layer on two streams at once and inside a captured HIP graph,
through the C ABI (needs an MI355X).

The library keeps no per-call state and never allocates, synchronises or
clears memory with a memset, so calls on different streams with their own
workspaces are independent, and a call can be recorded into a graph and
replayed on new input values.  The layer is deterministic, so every result is
compared bit for bit with the same call run alone on the default stream (the
oracle bounds that run's error in the parity tests).
"""
import pytest
import torch

from gpu_helpers import problem, to_device
from sparse_mixture_experts_moe_amd import binding as B
from workloads import CONFIGS, generate, shrink

pytestmark = pytest.mark.gpu

CFGS = {
    # about 8 rows per expert: the 32-row decode shape and the one-launch permutation
    "decode": shrink(CONFIGS["qwen_decode"], T=64, D=512, E=64, k=8, I=256, I_shared=256),
    # about 150 rows per expert: 256-row tiles, multi-block permutation, tile table
    "prefill": shrink(CONFIGS["qwen_prefill"], T=1200, D=256, E=64, k=8, I=128, I_shared=128),
    # fp8 weights
    "fp8": shrink(CONFIGS["ling_decode"], T=200, D=256, E=16, k=4, I=128, I_shared=128),
    # fp8 activations per 512-element sub-channel (quantiser launches, scale copies)
    "w8a8_sub": shrink(CONFIGS["ling_prefill"], T=700, D=1024, E=4, k=2, I=512, I_shared=512),
}
# modes of the graph cases: (act_quant, combine)
MODES = {"decode": (0, "auto"), "prefill": (0, "auto"), "fp8": (0, "auto"),
         "w8a8_sub": (B.MOE_ACT_QUANT_FP8_SUB, "auto"), "fused": (0, "fused")}
CFGS_OF = {"fused": "fp8"}


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _call(wl, ws, y, stream=None, mode=(0, "auto")):
    p = problem(wl.cfg, act_quant=mode[0], combine=mode[1])
    B.run_layer(p, wl.x, wl.w13, wl.w2, w_router=wl.wr, s13=wl.s13, s2=wl.s2,
                w13_shared=wl.w13s, s13_shared=wl.s13s, w2_shared=wl.w2s, s2_shared=wl.s2s,
                ws=ws, y=y, stream=stream)


def _buffers(wl, mode=(0, "auto")):
    need = B.moe_layer_workspace_size(problem(wl.cfg, act_quant=mode[0], combine=mode[1]))
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    y = torch.empty((wl.cfg.T, wl.cfg.D), dtype=wl.x.dtype, device="cuda")
    return ws, y


def test_layers_on_two_streams_at_once():
    wls = [to_device(generate(CFGS[n], seed=11)) for n in ("decode", "prefill", "fp8")]
    alone = []
    for wl in wls:
        ws, y = _buffers(wl)
        _call(wl, ws, y)
        torch.cuda.synchronize()
        alone.append(y.clone())
    # every layer twice, alternating between two streams, each call with its own
    # workspace and output, all enqueued before any is waited for
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    bufs = [_buffers(wl) for wl in wls for _ in range(2)]
    torch.cuda.synchronize()
    for rep in range(2):
        for i, wl in enumerate(wls):
            s = streams[(i + rep) % 2]
            ws, y = bufs[2 * i + rep]
            with torch.cuda.stream(s):
                _call(wl, ws, y, stream=s)
    torch.cuda.synchronize()
    for i in range(len(wls)):
        for rep in range(2):
            assert torch.equal(_bits(bufs[2 * i + rep][1]), _bits(alone[i])), (i, rep)


@pytest.mark.parametrize("name", ["decode", "prefill", "w8a8_sub", "fused"])
def test_layer_in_a_captured_graph(name):
    cfg = CFGS[CFGS_OF.get(name, name)]
    mode = MODES[name]
    wl = to_device(generate(cfg, seed=12))
    xs = [wl.x.clone()] + [torch.randn_like(wl.x, dtype=torch.float32).to(wl.x.dtype) for _ in range(3)]
    ws, y = _buffers(wl, mode)
    # eager results for every input (this also loads the kernels before capture)
    want = []
    for x in xs:
        wl.x.copy_(x)
        _call(wl, ws, y, mode=mode)
        torch.cuda.synchronize()
        want.append(y.clone())
    wl.x.copy_(xs[0])
    y.zero_()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _call(wl, ws, y, mode=mode)
    torch.cuda.synchronize()
    junk = torch.randn(512, 512, device="cuda")
    for rep in range(2):
        for i, x in enumerate(xs):
            wl.x.copy_(x)
            y.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(_bits(y), _bits(want[i])), (rep, i)
            # eager work on the same device between replays
            junk = torch.tanh(junk @ junk.T * 1e-3)
            torch.cuda.synchronize()
