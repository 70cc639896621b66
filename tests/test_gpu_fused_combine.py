"""The combine fused into the down projection against the separate combine
launch, through the C ABI (needs an MI355X).

Both paths sum a token's expert rows in fp32 in slot order with the shared
row last and round once, so the fused layer output must equal the separate
one bit for bit; whether a token is combined by the block that stored its
last row (the owner) must not show in the result.  Parity of the layer (with
the default, separate, combine) against the oracle is in test_gpu_parity.py;
bit-identity carries it over to the fused form."""
import pytest
import torch

from gpu_helpers import run_layer, to_device
from sparse_mixture_experts_moe_amd import binding as B
from test_gpu_parity import SMALL
from workloads import CONFIGS, generate, shrink

pytestmark = pytest.mark.gpu

# configurations whose down projection runs on the LDS-tiled kernel with bf16
# rows, so the fused combine must run (no separate combine launch)
FUSES = ("qwen_ragged", "gemma_like", "ling_fp8", "big_groups_bf16", "big_groups_fp8", "wide_fp8",
         "ling_decode_like")

QUANT = {
    "w8a8_wide": (shrink(CONFIGS["ling_prefill"], T=700, D=512, E=4, k=2, I=256, I_shared=128),
                  B.MOE_ACT_QUANT_FP8_ROW),
    "w8a8_decode": (shrink(CONFIGS["ling_decode"], T=96, D=512, E=32, k=4, I=256, I_shared=256),
                    B.MOE_ACT_QUANT_FP8_ROW),
    "w4a8_wide": (shrink(CONFIGS["ling_prefill_mxfp4"], T=700, D=512, E=4, k=2, I=256, I_shared=128),
                  B.MOE_ACT_QUANT_MXFP8),
    "w8a8_sub_tall": (shrink(CONFIGS["ling_prefill"], T=700, D=1024, E=4, k=2, I=512, I_shared=512),
                      B.MOE_ACT_QUANT_FP8_SUB),
    "w8a8_sub_decode": (shrink(CONFIGS["ling_decode"], T=96, D=1024, E=32, k=4, I=512, I_shared=512),
                        B.MOE_ACT_QUANT_FP8_SUB),
}


def _combine_launches(fn):
    """Run fn() with stage timing on; the number of separate combine launches."""
    B.moe_timing_read()
    B.moe_timing_enable(True)
    try:
        out = fn()
        torch.cuda.synchronize()
    finally:
        B.moe_timing_enable(False)
    return out, B.moe_timing_read()["combine"][1]


def _both(wl, act_quant=0):
    sep, n_sep = _combine_launches(lambda: run_layer(wl, act_quant=act_quant, combine="separate"))
    fus, n_fus = _combine_launches(lambda: run_layer(wl, act_quant=act_quant, combine="fused"))
    return sep, fus, n_sep, n_fus


def _assert_same(sep, fus, name):
    a, b = sep["y"], fus["y"]
    assert torch.isfinite(a.float()).all(), name
    diff = (a.view(torch.int16) != b.view(torch.int16))
    assert not diff.any(), f"{name}: fused combine differs from the separate one in {int(diff.sum())} elements"
    for key in ("topk_idx", "row_of_slot"):
        assert torch.equal(sep[key], fus[key]), (name, key)


@pytest.mark.parametrize("name", list(SMALL))
def test_fused_combine_bit_exact_small(name):
    cfg = SMALL[name]
    wl = to_device(generate(cfg, seed=11))
    sep, fus, n_sep, n_fus = _both(wl)
    _assert_same(sep, fus, name)
    assert n_sep == 1, name
    if name in FUSES:
        assert n_fus == 0, f"{name}: the fused combine did not run"


@pytest.mark.parametrize("name", list(QUANT))
def test_fused_combine_bit_exact_quantised(name):
    cfg, aq = QUANT[name]
    wl = to_device(generate(cfg, seed=12))
    sep, fus, n_sep, n_fus = _both(wl, aq)
    _assert_same(sep, fus, name)
    assert (n_sep, n_fus) == (1, 0), name


def test_fused_combine_repeated_calls_and_auto():
    """The arrival counters start from zero on every call (same workspace
    three times, starting from garbage), and the automatic choice is the
    separate combine (measured faster)."""
    cfg = SMALL["wide_fp8"]
    wl = to_device(generate(cfg, seed=13))
    p = B.make_problem(cfg.T, cfg.D, cfg.E, cfg.k, cfg.I, cfg.I_shared, cfg.act, cfg.act_shared,
                       cfg.act_dtype, cfg.w_dtype, cfg.shared_w_dtype, combine="fused")
    ws = torch.full((B.moe_layer_workspace_size(p),), 0x5A, dtype=torch.uint8, device="cuda")
    kw = dict(w_router=wl.wr, s13=wl.s13, s2=wl.s2, w13_shared=wl.w13s, s13_shared=wl.s13s,
              w2_shared=wl.w2s, s2_shared=wl.s2s)
    ys = [B.run_layer(p, wl.x, wl.w13, wl.w2, ws=ws, **kw)["y"].clone() for _ in range(3)]
    torch.cuda.synchronize()
    sep = run_layer(wl, combine="separate", want=())
    for y in ys:
        assert torch.equal(y.view(torch.int16), sep["y"].view(torch.int16))
    auto, n_auto = _combine_launches(lambda: run_layer(wl, want=()))
    assert n_auto == 1
    assert torch.equal(auto["y"].view(torch.int16), sep["y"].view(torch.int16))


@pytest.mark.parametrize("name", ["qwen_decode", "qwen_prefill", "gemma", "ling_decode", "ling_prefill"])
def test_fused_combine_bit_exact_full_size(name):
    cfg = CONFIGS[name]
    torch.cuda.set_device(0)
    wl = generate(cfg, seed=0, weight_device="cuda")
    wl.x, wl.wr = wl.x.cuda(), wl.wr.cuda()
    want = ("topk_idx_out", "row_of_slot_out")
    sep, n_sep = _combine_launches(lambda: run_layer(wl, combine="separate", want=want))
    fus, n_fus = _combine_launches(lambda: run_layer(wl, combine="fused", want=want))
    _assert_same(sep, fus, name)
    assert (n_sep, n_fus) == (1, 0), name
    del wl, sep, fus
    torch.cuda.empty_cache()


def test_fused_combine_stable_over_many_calls():
    """Twenty fused calls in a row on a layer whose tokens' rows come from
    blocks on every XCD: each output equals the separate combine's bit for bit
    (the owner's reads see every other block's rows each time)."""
    cfg = shrink(CONFIGS["ling_decode"], T=384, D=1024, E=32, k=8, I=256, I_shared=256)
    wl = to_device(generate(cfg, seed=14))
    sep = run_layer(wl, combine="separate", want=())["y"]
    for i in range(20):
        fus = run_layer(wl, combine="fused", want=())["y"]
        assert torch.equal(fus.view(torch.int16), sep.view(torch.int16)), f"call {i}"
