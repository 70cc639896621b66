"""Dynamic per-token fp8 activations (W8A8) through the C ABI vs the oracle
(needs an MI355X).

The HIP path is compared with oracle/actquant.py, which performs the same
quantisation: the codes and scales of moe_quantize_rows bit for bit, the layer
within the fp8 tolerance.  The difference of the W8A8 layer from the exact
layer (the quantisation itself, a few per cent) is pinned on the CPU.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import check_matched, f64, oracle_inputs, run_layer, to_device
from oracle.actquant import dequantize_rows, expert_ffn_w8a8, layer_w8a8, quantize_rows
from oracle.formats import decode, fp8_e4m3fn_table
from oracle.moe import router_logits
from sparse_mixture_experts_moe_amd import binding as B
from workloads import CONFIGS, generate, shrink, to_bits

pytestmark = pytest.mark.gpu

AQ = B.MOE_ACT_QUANT_FP8_ROW
TABLE = fp8_e4m3fn_table()
ROUTING = ("idx", "counts", "offsets", "row_token", "row_of_slot")


def _same_codes(got: np.ndarray, want: np.ndarray) -> bool:
    """Equal codes, where +0 and -0 (0x00 / 0x80) count as the same value."""
    return bool(np.all((got == want) | ((TABLE[got] == 0) & (TABLE[want] == 0))))


@pytest.mark.parametrize("rows,cols,lda", [(1, 8, 8), (37, 256, 264), (300, 2048, 2048),
                                           (16, 8192, 8192), (5, 16384, 16384)])
def test_quantize_rows_bit_exact(rows, cols, lda):
    rng = np.random.default_rng(rows * 7 + cols)
    a = rng.standard_normal((rows, lda)).astype(np.float32)
    a *= np.exp2(rng.integers(-20, 20, size=(rows, 1))).astype(np.float32)   # per-row magnitudes
    if rows > 2:
        a[1] = 0.0                                                        # zero row -> scale 1
        a[2, :cols] = -a[2, :cols]
    if rows > 3:
        # a row on the fp8 grid with a power-of-two scale and values at exact
        # midpoints between codes, so ties must go to the even code
        codes = rng.integers(0, 0x7E, size=cols)
        mids = (TABLE[codes] + TABLE[codes + 1]) / 2
        mids[0] = 448.0
        a[3, :cols] = (mids * 2.0 ** -5).astype(np.float32)
    if rows > 6:
        # exact midpoints again, reached through scales 3, 5 and 7 (the row
        # maximum 448 s): the quotients x / s are ties that a product with
        # the rounded reciprocal of s misses by an ulp
        for rr, m in ((4, 3.0), (5, 5.0), (6, 7.0)):
            codes = rng.integers(0, 0x7E, size=cols)
            row = ((TABLE[codes] + TABLE[codes + 1]) / 2 * m).astype(np.float32)
            row *= rng.choice([-1.0, 1.0], size=cols).astype(np.float32)
            row[0] = 448.0 * m
            keep = torch.from_numpy(row).to(torch.bfloat16).float().numpy() == row
            a[rr, :cols] = np.where(keep, row, 0.0)
            assert keep.mean() > 0.9
    at = torch.from_numpy(a).to(torch.bfloat16).cuda()
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    s = torch.empty(rows, dtype=torch.float32, device="cuda")
    B.moe_quantize_rows(at, rows, cols, lda, q, s)
    torch.cuda.synchronize()
    ref_q, ref_s = quantize_rows(decode(to_bits(at.cpu())[:, :cols], "bf16"))
    assert np.array_equal(s.cpu().numpy(), ref_s)
    assert _same_codes(q.cpu().numpy(), ref_q)


SMALL = {
    "ling_fp8": shrink(CONFIGS["ling_decode"], T=130, D=256, E=16, k=8, I=128, I_shared=128),
    # more than 256 rows per expert: 128-row tiles with ragged tails
    "big_groups_fp8": shrink(CONFIGS["ling_prefill"], T=1030, D=384, E=4, k=2, I=256, I_shared=128),
    "no_shared": shrink(CONFIGS["ling_decode"], T=77, D=128, E=8, k=3, I=256, I_shared=0),
    # about 24 rows per expert: the 64-row decode shape, routed and shared sets
    "decode_fp8": shrink(CONFIGS["ling_decode"], T=96, D=256, E=32, k=8, I=128, I_shared=128),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_w8a8_small(name):
    cfg = SMALL[name]
    wl = to_device(generate(cfg, seed=4))
    x, wr, expert, shared = oracle_inputs(wl)
    ref = layer_w8a8(x, wr, cfg.k, expert, shared, cfg.act, cfg.act_shared)
    res = run_layer(wl, logits_in=torch.from_numpy(ref["logits"]).cuda(), act_quant=AQ)
    got = {"idx": res["topk_idx"], "counts": res["counts"], "offsets": res["offsets"],
           "row_token": res["row_token"], "row_of_slot": res["row_of_slot"]}
    for n in ROUTING:
        assert np.array_equal(got[n].cpu().numpy(), np.asarray(ref[n]).reshape(got[n].shape)), n
    check_matched(f64(res["y"]), ref["y"], f"w8a8 {name}")


def test_grouped_ffn_w8a8_entry():
    """One dense group through moe_grouped_ffn with fp8 activations."""
    cfg = SMALL["big_groups_fp8"]
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
    xd = dequantize_rows(*quantize_rows(x))
    ref = expert_ffn_w8a8(xd, *shared, cfg.act_shared)
    check_matched(f64(out), ref, "w8a8 grouped FFN, shared branch")


@pytest.mark.parametrize("name", ["ling_decode", "ling_prefill"])
def test_full_size_w8a8(name):
    """Every element of y at the benchmark sizes against the matched oracle."""
    cfg = CONFIGS[name]
    print(f"[full-size w8a8] {name}: generating on GPU", flush=True)
    wl = generate(cfg, seed=0, weight_device="cuda")
    to_device(wl)
    x, wr, expert, shared = oracle_inputs(wl)
    logits_ref = router_logits(x, wr)
    print(f"[full-size w8a8] {name}: running moe_layer", flush=True)
    res = run_layer(wl, logits_in=torch.from_numpy(logits_ref).cuda(), act_quant=AQ)
    y = f64(res["y"])
    print(f"[full-size w8a8] {name}: oracle, whole layer", flush=True)
    ref = layer_w8a8(x, wr, cfg.k, expert, shared, cfg.act, cfg.act_shared, logits_in=logits_ref)
    for n in ROUTING:
        got = {"idx": res["topk_idx"], "counts": res["counts"], "offsets": res["offsets"],
               "row_token": res["row_token"], "row_of_slot": res["row_of_slot"]}[n]
        assert np.array_equal(got.cpu().numpy(), np.asarray(ref[n]).reshape(got.shape)), n
    check_matched(y, ref["y"], f"full-size w8a8 {name}")
    del wl, res, ref, y
    torch.cuda.empty_cache()
