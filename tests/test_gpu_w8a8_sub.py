"""fp8 activations with one scale per 512-element sub-channel through the C
ABI vs the oracle (needs an MI355X).

The sub-channel activation quantisation of the fp8 grouped matmul ("Qwen 3.5
MoE on Ironwood" page, MoE track, GMM v2).  The HIP path is compared with
oracle/actquant.py at width 512, which performs the same quantisation: the
codes and scales of moe_quantize_subchannel bit for bit, the layer within the
fp8 tolerance of the matched comparison.  What the quantisation itself does
(per-slice scales, boundaries, error bound) is pinned on the CPU.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import check_matched, f64, oracle_inputs, run_layer, to_device
from oracle.actquant import expert_ffn_w8a8, layer_w8a8, quantize_dequantize, quantize_subchannel
from oracle.formats import decode, fp8_e4m3fn_table
from oracle.moe import router_logits
from sparse_mixture_experts_moe_amd import binding as B
from workloads import CONFIGS, generate, shrink, to_bits

pytestmark = pytest.mark.gpu

AQ = B.MOE_ACT_QUANT_FP8_SUB
W = B.MOE_SUBCHANNEL
TABLE = fp8_e4m3fn_table()
ROUTING = ("idx", "counts", "offsets", "row_token", "row_of_slot")


def _same_codes(got: np.ndarray, want: np.ndarray) -> bool:
    """Equal codes, where +0 and -0 (0x00 / 0x80) count as the same value."""
    return bool(np.all((got == want) | ((TABLE[got] == 0) & (TABLE[want] == 0))))


@pytest.mark.parametrize("rows,cols,lda", [(1, 512, 512), (37, 1024, 1032), (300, 2048, 2048),
                                           (16, 8192, 8192), (5, 16384, 16384)])
def test_quantize_subchannel_bit_exact(rows, cols, lda):
    rng = np.random.default_rng(rows * 11 + cols)
    a = rng.standard_normal((rows, lda)).astype(np.float32)
    # per-slice magnitudes 2^-20 .. 2^20
    mags = np.exp2(rng.integers(-20, 20, size=(rows, (lda + W - 1) // W))).astype(np.float32)
    a *= np.repeat(mags, W, axis=1)[:, :lda]
    if rows > 2:
        a[1, W // 2:W + 7] = 0.0           # a zero run across a slice boundary
        if cols >= 2 * W:
            a[2, W:2 * W] = 0.0            # a zero slice -> scale 1
    if rows > 3:
        # a slice on the fp8 grid with a power-of-two scale, values at exact
        # midpoints between codes: ties must go to the even code
        codes = rng.integers(0, 0x7E, size=W)
        mids = (TABLE[codes] + TABLE[codes + 1]) / 2
        mids[0] = 448.0
        a[3, :W] = (mids * 2.0 ** -5).astype(np.float32)
    if rows > 4:
        # exact midpoints through the slice scales 3, 5 and 7 (slice maximum
        # 448 s), one slice each: ties that a product with the rounded
        # reciprocal of s misses by an ulp
        for u, m in zip(range(cols // W), (3.0, 5.0, 7.0)):
            codes = rng.integers(0, 0x7E, size=W)
            sl = ((TABLE[codes] + TABLE[codes + 1]) / 2 * m).astype(np.float32)
            sl *= rng.choice([-1.0, 1.0], size=W).astype(np.float32)
            sl[0] = 448.0 * m
            keep = torch.from_numpy(sl).to(torch.bfloat16).float().numpy() == sl
            a[4, u * W:(u + 1) * W] = np.where(keep, sl, 0.0)
            assert keep.mean() > 0.9
    at = torch.from_numpy(a).to(torch.bfloat16).cuda()
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    s = torch.empty((cols // W, rows), dtype=torch.float32, device="cuda")
    B.moe_quantize_subchannel(at, rows, cols, lda, q, s)
    torch.cuda.synchronize()
    ref_q, ref_s = quantize_subchannel(decode(to_bits(at.cpu())[:, :cols], "bf16"), W)
    assert np.array_equal(s.cpu().numpy().T, ref_s)
    assert _same_codes(q.cpu().numpy(), ref_q)


SMALL = {
    # about 65 rows per expert: 256-row tiles, routed and shared sets
    "ling_sub": shrink(CONFIGS["ling_decode"], T=130, D=1024, E=16, k=8, I=512, I_shared=512),
    # more than 256 rows per expert: several 256-row tiles with ragged tails
    "big_groups_sub": shrink(CONFIGS["ling_prefill"], T=1030, D=1024, E=4, k=2, I=512, I_shared=512),
    # about 24 rows per expert: the 64-row decode shape
    "decode_sub": shrink(CONFIGS["ling_decode"], T=96, D=1024, E=32, k=8, I=512, I_shared=512),
    "no_shared_sub": shrink(CONFIGS["ling_decode"], T=77, D=512, E=8, k=3, I=1024, I_shared=0),
}


def _run_and_check(cfg, wl, what, x_scale=None):
    x, wr, expert, shared = oracle_inputs(wl)
    ref = layer_w8a8(x, wr, cfg.k, expert, shared, cfg.act, cfg.act_shared, width=W)
    res = run_layer(wl, logits_in=torch.from_numpy(ref["logits"]).cuda(), act_quant=AQ)
    got = {"idx": res["topk_idx"], "counts": res["counts"], "offsets": res["offsets"],
           "row_token": res["row_token"], "row_of_slot": res["row_of_slot"]}
    for n in ROUTING:
        assert np.array_equal(got[n].cpu().numpy(), np.asarray(ref[n]).reshape(got[n].shape)), n
    check_matched(f64(res["y"]), ref["y"], what)


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_sub_small(name):
    cfg = SMALL[name]
    wl = to_device(generate(cfg, seed=4))
    _run_and_check(cfg, wl, f"w8a8 sub-channel {name}")


def test_layer_sub_slices_of_very_different_magnitude():
    """Token rows whose 512-element slices differ in magnitude by up to 2^32
    (and some all-zero slices): the slice scales' powers of two go to the
    matrix cores and the accumulators are rescaled between slices, so every
    output still matches the oracle."""
    cfg = SMALL["ling_sub"]
    wl = generate(cfg, seed=6)
    rng = np.random.default_rng(6)
    f = np.exp2(rng.integers(-16, 17, size=(cfg.T, cfg.D // W))).astype(np.float32)
    f[rng.random(f.shape) < 0.05] = 0.0
    x = wl.x.float() * torch.from_numpy(np.repeat(f, W, axis=1))
    wl.x = x.to(torch.bfloat16)
    _run_and_check(cfg, to_device(wl), "w8a8 sub-channel, mixed slice magnitudes")


def test_grouped_ffn_sub_entry():
    """One dense group through moe_grouped_ffn with sub-channel fp8 activations."""
    cfg = SMALL["big_groups_sub"]
    wl = to_device(generate(cfg, seed=9))
    x, _, _, shared = oracle_inputs(wl)
    p = B.make_problem(cfg.T, cfg.D, 1, 1, cfg.I_shared, 0, cfg.act_shared, cfg.act_shared,
                       cfg.act_dtype, cfg.shared_w_dtype, cfg.shared_w_dtype, act_quant=AQ)
    h = torch.empty((cfg.T, cfg.I_shared), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((cfg.T, cfg.D), dtype=torch.bfloat16, device="cuda")
    n = B.moe_grouped_ffn_workspace_size(p, 1, cfg.T)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    B.moe_grouped_ffn(p, 1, cfg.T, wl.x, None, torch.tensor([0, cfg.T], dtype=torch.int32).cuda(),
                      wl.w13s, wl.s13s, wl.w2s, wl.s2s, h, out, ws, n)
    torch.cuda.synchronize()
    ref = expert_ffn_w8a8(quantize_dequantize(x, W), *shared, cfg.act_shared, W)
    check_matched(f64(out), ref, "w8a8 sub-channel grouped FFN, shared branch")


@pytest.mark.parametrize("name", ["ling_decode", "ling_prefill"])
def test_full_size_sub(name):
    """Every element of y at the benchmark sizes against the matched oracle."""
    cfg = CONFIGS[name]
    print(f"[full-size w8a8 sub-channel] {name}: generating on GPU", flush=True)
    wl = generate(cfg, seed=0, weight_device="cuda")
    to_device(wl)
    x, wr, expert, shared = oracle_inputs(wl)
    logits_ref = router_logits(x, wr)
    print(f"[full-size w8a8 sub-channel] {name}: running moe_layer", flush=True)
    res = run_layer(wl, logits_in=torch.from_numpy(logits_ref).cuda(), act_quant=AQ)
    y = f64(res["y"])
    print(f"[full-size w8a8 sub-channel] {name}: oracle, whole layer", flush=True)
    ref = layer_w8a8(x, wr, cfg.k, expert, shared, cfg.act, cfg.act_shared, logits_in=logits_ref, width=W)
    for n in ROUTING:
        got = {"idx": res["topk_idx"], "counts": res["counts"], "offsets": res["offsets"],
               "row_token": res["row_token"], "row_of_slot": res["row_of_slot"]}[n]
        assert np.array_equal(got.cpu().numpy(), np.asarray(ref[n]).reshape(got.shape)), n
    check_matched(y, ref["y"], f"full-size w8a8 sub-channel {name}")
    del wl, res, ref, y
    torch.cuda.empty_cache()
