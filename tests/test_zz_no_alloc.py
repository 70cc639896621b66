"""moe_layer_noalloc, the entry point that allocates nothing, against moe_layer
through the C ABI (needs an MI355X): the same launches on the same inputs, so
the outputs must be identical bit for bit, on two calls in a row (the second
smaller, so it runs on what the first left in the library's array)."""
import numpy as np
import pytest
import torch

from gpu_helpers import problem, to_device
from sparse_mixture_experts_moe_amd import binding as B
from workloads import CONFIGS, generate, shrink

pytestmark = pytest.mark.gpu


def _args(wl, y, idx):
    return B.layer_args(x=wl.x, w_router=wl.wr, w13=wl.w13, s13=wl.s13, w2=wl.w2, s2=wl.s2,
                        w13_shared=wl.w13s, s13_shared=wl.s13s, w2_shared=wl.w2s, s2_shared=wl.s2s,
                        y=y, topk_idx_out=idx)


def _outputs(cfg, wl):
    y = torch.empty((cfg.T, cfg.D), dtype=wl.x.dtype, device="cuda")
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    return y, idx


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_noalloc_matches_moe_layer_on_two_calls():
    # the Ling decode batch (fp8 weights, about 106 MiB of workspace), then a
    # smaller bf16 decode batch
    cases = [(CONFIGS["ling_decode"], 0),
             (shrink(CONFIGS["qwen_decode"], T=40, D=512, E=32, k=4, I=256, I_shared=256), 3)]
    runs = []
    for cfg, seed in cases:
        print(f"[noalloc] reference moe_layer: {cfg.name} T={cfg.T} D={cfg.D} E={cfg.E}", flush=True)
        wl = to_device(generate(cfg, seed=seed, weight_device="cuda"))
        p = problem(cfg)
        need = B.moe_layer_workspace_size(p)
        assert need <= B.moe_layer_noalloc_max_bytes()
        y_ref, idx_ref = _outputs(cfg, wl)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        B.moe_layer(p, _args(wl, y_ref, idx_ref), ws, need)
        torch.cuda.synchronize()
        del ws
        runs.append((cfg, wl, p, y_ref, idx_ref))
    # two allocation-free calls in a row, the second smaller
    got = []
    for cfg, wl, p, _, _ in runs:
        print(f"[noalloc] moe_layer_noalloc: {cfg.name}", flush=True)
        y, idx = _outputs(cfg, wl)
        B.moe_layer_noalloc(p, _args(wl, y, idx))
        got.append((y, idx))
    torch.cuda.synchronize()
    for (cfg, _, _, y_ref, idx_ref), (y, idx) in zip(runs, got):
        assert torch.equal(idx, idx_ref), cfg.name
        assert torch.equal(_bits(y), _bits(y_ref)), cfg.name
        assert np.isfinite(y.float().cpu().numpy()).all()


def test_noalloc_rejects_a_problem_larger_than_its_array():
    cfg = CONFIGS["ling_prefill"]   # about 2.9 GiB of workspace
    p = problem(cfg)
    assert B.moe_layer_workspace_size(p) > B.moe_layer_noalloc_max_bytes()
    fake = 4096   # never dereferenced: the size check comes first
    args = B.layer_args(x=fake, w_router=fake, w13=fake, s13=fake, w2=fake, s2=fake, w13_shared=fake,
                        s13_shared=fake, w2_shared=fake, s2_shared=fake, y=fake)
    with pytest.raises(B.MoeError) as e:
        B.moe_layer_noalloc(p, args)
    assert e.value.status == B.MOE_ERR_WORKSPACE
