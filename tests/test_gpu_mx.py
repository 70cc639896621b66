"""MXFP4 weights with MXFP8 activations (W4A8) through the C ABI vs the oracle
(needs an MI355X).

The HIP path is compared with oracle/mx.py, which performs the same block
quantisation: moe_quantize_rows_mx's codes and E8M0 scales bit for bit, the
layer within the fp8 tolerance (the GPU's fp32 sums and the oracle's float64
ones may round a stored bf16 h, and so an MXFP8 code of h, differently).  How
far the W4A8 layer is from the exact one is pinned on the CPU.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import check_matched, f64, oracle_inputs, rel_err, run_layer, to_device
from oracle.actquant import round_bf16
from oracle.formats import decode, fp8_e4m3fn_table
from oracle.moe import router_logits
from oracle.mx import expert_ffn_w4a8, layer_w4a8, mx_quantize, mx_round_trip
from sparse_mixture_experts_moe_amd import binding as B
from workloads import CONFIGS, generate, shrink, to_bits

pytestmark = pytest.mark.gpu

AQ = B.MOE_ACT_QUANT_MXFP8
TABLE = fp8_e4m3fn_table()
ROUTING = ("idx", "counts", "offsets", "row_token", "row_of_slot")


def _same_codes(got: np.ndarray, want: np.ndarray) -> bool:
    """Equal codes, where +0 and -0 (0x00 / 0x80) count as the same value."""
    return bool(np.all((got == want) | ((TABLE[got] == 0) & (TABLE[want] == 0))))


def _scales_by_row(s: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """[cols/128][rows][4] scale bytes -> [rows][cols/32]."""
    return s.reshape(cols // 128, rows, 4).transpose(1, 0, 2).reshape(rows, cols // 32)


def _bf16_values(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)


@pytest.mark.parametrize("rows,cols,lda", [(1, 128, 128), (37, 256, 264), (300, 2048, 2048),
                                           (16, 8192, 8192), (5, 16384, 16384)])
def test_quantize_rows_mx_bit_exact(rows, cols, lda):
    rng = np.random.default_rng(rows * 11 + cols)
    a = rng.standard_normal((rows, lda)).astype(np.float32)
    # per-row and per-block magnitudes, so neighbouring blocks get other scales
    a *= np.exp2(rng.integers(-20, 20, size=(rows, 1))).astype(np.float32)
    a[:, :cols] *= np.repeat(np.exp2(rng.integers(-6, 6, size=(rows, cols // 32))), 32, axis=1)
    if rows > 4:
        a[1] = 0.0                                          # zero blocks: scale code 0
        a[2, :32] = 0.0
        a[2, 32:64] = -a[2, 32:64]
        # bf16 subnormals: floor(log2 amax) - 8 below -127 clamps to -127
        a[3, :cols] = rng.choice([-3.0, -1.0, 1.0, 2.0, 5.0], size=cols) * 2.0 ** -133
        # block on the scaled e4m3 grid with ties between neighbouring codes
        # (scale 2^-5: block peak 448 * 2^-5 sets floor(log2) - 8 = -5)
        codes = rng.integers(0, 0x7E, size=cols)
        mids = (TABLE[codes] + TABLE[codes + 1]) / 2
        mids[::32] = 448.0
        a[4, :cols] = mids * 2.0 ** -5
    at = _bf16_values(a).cuda()
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    s = torch.empty(rows * cols // 32, dtype=torch.uint8, device="cuda")
    B.moe_quantize_rows_mx(at, rows, cols, lda, q, s)
    torch.cuda.synchronize()
    ref_q, ref_s = mx_quantize(decode(to_bits(at.cpu())[:, :cols], "bf16"), "e4m3")
    assert np.array_equal(_scales_by_row(s.cpu().numpy(), rows, cols), ref_s)
    assert _same_codes(q.cpu().numpy(), ref_q)
    if rows > 4:
        assert np.all(ref_s[1] == 0) and np.all(ref_s[3] == 0)


SMALL = {
    "ling_mx": shrink(CONFIGS["ling_decode_mxfp4"], T=130, D=256, E=16, k=8, I=128, I_shared=128),
    # more than 256 rows per expert: 128-row tiles with ragged tails, K = 384 (3 stages)
    "big_groups_mx": shrink(CONFIGS["ling_prefill_mxfp4"], T=1030, D=384, E=4, k=2, I=256, I_shared=128),
    "no_shared_mx": shrink(CONFIGS["ling_decode_mxfp4"], T=77, D=128, E=8, k=3, I=256, I_shared=0),
    # about 24 rows per expert: the 64-row decode shape, routed and shared sets
    "decode_mx": shrink(CONFIGS["ling_decode_mxfp4"], T=96, D=256, E=32, k=8, I=128, I_shared=128),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_w4a8_small(name):
    cfg = SMALL[name]
    print(f"[w4a8] {name}: T={cfg.T} D={cfg.D} E={cfg.E} k={cfg.k} I={cfg.I}", flush=True)
    wl = to_device(generate(cfg, seed=4))
    x, wr, expert, shared = oracle_inputs(wl)
    ref = layer_w4a8(x, wr, cfg.k, expert, shared, cfg.act, cfg.act_shared)
    res = run_layer(wl, logits_in=torch.from_numpy(ref["logits"]).cuda(), act_quant=AQ)
    got = {"idx": res["topk_idx"], "counts": res["counts"], "offsets": res["offsets"],
           "row_token": res["row_token"], "row_of_slot": res["row_of_slot"]}
    for n in ROUTING:
        assert np.array_equal(got[n].cpu().numpy(), np.asarray(ref[n]).reshape(got[n].shape)), n
    check_matched(f64(res["y"]), ref["y"], f"w4a8 {name}")


def test_grouped_ffn_w4a8_entry():
    """One dense group through moe_grouped_ffn with MXFP8 activations; h is
    checked too (before its own quantisation)."""
    cfg = SMALL["big_groups_mx"]
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
    xd = mx_round_trip(x, "e4m3")
    w13, _, w2, _ = shared
    gu = xd @ w13.T
    I = cfg.I_shared
    from oracle.moe import ACTS
    h_ref = round_bf16(ACTS[cfg.act_shared](gu[:, :I]) * gu[:, I:])
    assert rel_err(f64(h), h_ref) <= 1e-2
    ref = expert_ffn_w4a8(xd, w13, w2, cfg.act_shared)
    check_matched(f64(out), ref, "w4a8 grouped FFN, shared branch")


@pytest.mark.parametrize("name", ["ling_decode_mxfp4", "ling_prefill_mxfp4"])
def test_full_size_w4a8(name):
    """Every element of y at the benchmark sizes against the matched oracle."""
    cfg = CONFIGS[name]
    print(f"[full-size w4a8] {name}: generating on GPU", flush=True)
    wl = generate(cfg, seed=0, weight_device="cuda")
    to_device(wl)
    x, wr, expert, shared = oracle_inputs(wl)
    logits_ref = router_logits(x, wr)
    print(f"[full-size w4a8] {name}: running moe_layer", flush=True)
    res = run_layer(wl, logits_in=torch.from_numpy(logits_ref).cuda(), act_quant=AQ)
    y = f64(res["y"])
    print(f"[full-size w4a8] {name}: oracle, whole layer", flush=True)
    ref = layer_w4a8(x, wr, cfg.k, expert, shared, cfg.act, cfg.act_shared, logits_in=logits_ref)
    got = {"idx": res["topk_idx"], "counts": res["counts"], "offsets": res["offsets"],
           "row_token": res["row_token"], "row_of_slot": res["row_of_slot"]}
    for n in ROUTING:
        assert np.array_equal(got[n].cpu().numpy(), np.asarray(ref[n]).reshape(got[n].shape)), n
    check_matched(y, ref["y"], f"full-size w4a8 {name}")
    del wl, res, ref, y
    torch.cuda.empty_cache()
