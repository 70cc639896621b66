"""HIP path vs the CPU oracle, through the C ABI (needs an MI355X)."""
import numpy as np
import pytest
import torch

from gpu_helpers import (f64, oracle_inputs, oracle_layer, problem, rel_err, run_layer, to_device,
                         tol_for)
from oracle.actquant import encode_e4m3fn
from oracle.formats import fp8_e4m3fn_table
from oracle.moe import layer, layer_tokens, permute, router_logits, topk_softmax
from sparse_mixture_experts_moe_amd import binding as B
from workloads import CONFIGS, generate, shrink

pytestmark = pytest.mark.gpu

ROUTING = ("idx", "counts", "offsets", "row_token", "row_of_slot")

SMALL = {
    "tiny_fp32": CONFIGS["tiny_fp32"],
    "qwen_ragged": shrink(CONFIGS["qwen_decode"], T=300, D=256, E=16, k=4, I=128, I_shared=128),
    "qwen_decode_like": shrink(CONFIGS["qwen_decode"], T=64, D=512, E=64, k=10, I=128, I_shared=128),
    "qwen_zipf": shrink(CONFIGS["qwen_prefill"], T=520, D=256, E=32, k=10, I=64, I_shared=64),
    "gemma_like": shrink(CONFIGS["gemma"], T=200, D=320, E=16, k=8, I=192, I_shared=320),
    "ling_fp8": shrink(CONFIGS["ling_decode"], T=130, D=256, E=16, k=8, I=128, I_shared=128),
    "fp32_ragged": shrink(CONFIGS["tiny_fp32"], T=77, D=192, E=12, k=3, I=64),
    # more than 256 rows per expert on average: 256-row LDS tiles with ragged tails
    "big_groups_bf16": shrink(CONFIGS["qwen_prefill"], T=1100, D=256, E=4, k=2, I=192, I_shared=128,
                              zipf=False),
    "big_groups_fp8": shrink(CONFIGS["ling_prefill"], T=1030, D=320, E=4, k=2, I=128, I_shared=192),
    # fp8 weights, about 550 rows per expert, D and I filling whole 512-wide
    # blocks: the 128 x 512 fp8 shape over several tiles per expert with
    # ragged last tiles, and K = D, I not a multiple of six stages
    "wide_fp8": shrink(CONFIGS["ling_prefill"], T=1100, D=1024, E=4, k=2, I=768, I_shared=256),
    # fp8 weights, about 12 rows per expert with Zipf-skewed loads (empty experts
    # and experts over 32 rows): the automatic policy's 32-row tiled shape
    "ling_decode_like": shrink(CONFIGS["ling_decode"], T=200, D=512, E=64, k=4, I=256, I_shared=256,
                               zipf=True),
    # bf16 decode with K = D = 2304 on the gate/up projection: the 32-row
    # shape's 256-deep stages (9 of them), 128-deep ones on the down projection
    "qwen_decode_deep": shrink(CONFIGS["qwen_decode"], T=40, D=2304, E=32, k=6, I=384, I_shared=128),
    # about 150 rows per expert with D = 512: 256-row tiles for gate/up, the
    # down projection on 128 x 512 tiles from a tile table of its own
    "qwen_prefill_like": shrink(CONFIGS["qwen_prefill"], T=600, D=512, E=32, k=8, I=128, I_shared=128),
    # bf16 routed experts with an fp8 shared expert: one launch per weight dtype
    "mixed_dtypes": shrink(CONFIGS["qwen_prefill"], T=600, D=512, E=32, k=8, I=128, I_shared=128,
                           shared_w_dtype="fp8"),
}


def _check_routing(res, ref, w_rtol=1e-6):
    got = {"idx": res["topk_idx"], "counts": res["counts"], "offsets": res["offsets"],
           "row_token": res["row_token"], "row_of_slot": res["row_of_slot"]}
    for n in ROUTING:
        g = got[n].cpu().numpy()
        r = np.asarray(ref[n]).reshape(g.shape)
        assert np.array_equal(g, r), f"{n} differs at {np.argwhere(g != r)[:5].tolist()}"
    w = res["topk_w"].cpu().numpy().astype(np.float64)
    wr = np.asarray(ref["w"], np.float64)
    assert np.max(np.abs(w - wr) / np.abs(wr)) <= w_rtol


# ------------------------------------------------------------------ formats
def test_fp8_decode_all_256_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).cuda()
    out = torch.empty(256, dtype=torch.int16, device="cuda")
    B.moe_debug_fp8_to_bf16(codes, out, 256)
    torch.cuda.synchronize()
    got = f64(out.view(torch.bfloat16))
    ref = fp8_e4m3fn_table()
    nan = np.isnan(ref)
    assert np.all(np.isnan(got[nan]))
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_fp8_encode_against_the_format():
    """The activation quantisers' fp32 -> e4m3fn encoder against the oracle's
    (nearest value, ties to the even code, saturating at 448): every code's
    value and every midpoint between neighbouring codes with four fp32 ulps on
    either side, 2^22 values spread over 2^-24 .. 2^10, values past 448, both
    signs."""
    pos = fp8_e4m3fn_table()[:0x7F].astype(np.float32)            # 0 .. 448
    base = np.concatenate([pos, ((pos[:-1].astype(np.float64) + pos[1:]) / 2).astype(np.float32)])
    vals, up, dn = [base], base.copy(), base.copy()
    for _ in range(4):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(-np.inf))
        vals += [up, dn]
    rng = np.random.default_rng(5)
    n = 1 << 22
    vals.append((rng.standard_normal(n) * np.exp2(rng.uniform(-24, 10, n))).astype(np.float32))
    vals.append(np.array([448.0, 460.0, 480.0, 1.0e30, 2.0 ** -10, 2.0 ** -11], np.float32))
    v = np.concatenate(vals)
    v = np.concatenate([v, -v])
    got = torch.empty(v.size, dtype=torch.uint8, device="cuda")
    B.moe_debug_f32_to_fp8(torch.from_numpy(v).cuda(), got, v.size)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    ref = encode_e4m3fn(v)
    same = (got == ref) | (((got & 0x7F) == 0) & ((ref & 0x7F) == 0))   # +0 and -0 alike
    assert same.all(), [(float(x), hex(int(g)), hex(int(r))) for x, g, r in
                        zip(v[~same][:8], got[~same][:8], ref[~same][:8])]


# ------------------------------------------------------------------ whole layer, small
@pytest.mark.parametrize("policy", ["stream", "lds", "auto"])
@pytest.mark.parametrize("name", list(SMALL))
def test_layer_small_with_oracle_logits(name, policy):
    cfg = SMALL[name]
    wl = to_device(generate(cfg, seed=1))
    ref = oracle_layer(wl)
    logits_in = torch.from_numpy(ref["logits"]).cuda()
    res = run_layer(wl, policy, logits_in=logits_in)
    _check_routing(res, ref)
    err = rel_err(f64(res["y"]), ref["y"])
    assert err <= tol_for(cfg), f"{name}/{policy}: rel err {err:.3e}"


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_small_on_device_logits(name):
    cfg = SMALL[name]
    wl = to_device(generate(cfg, seed=2))
    ref = oracle_layer(wl)
    res = run_layer(wl)
    lg, lr = f64(res["logits"]), ref["logits"].astype(np.float64)
    assert np.max(np.abs(lg - lr)) <= 1e-5 * max(1.0, np.max(np.abs(lr)))
    same = np.all(np.sort(res["topk_idx"].cpu().numpy(), 1) == np.sort(ref["idx"], 1), axis=1)
    assert same.mean() >= 0.99
    if same.all():
        # the weights come from the device's own logits, which differ from the
        # oracle's by rounding: |dw/w| <= 2 max|dl| (softmax over the top-k)
        dl = float(np.max(np.abs(lg - lr)))
        _check_routing(res, ref, w_rtol=1e-6 + 2.5 * dl)
        assert rel_err(f64(res["y"]), ref["y"]) <= tol_for(cfg)
    else:
        assert rel_err(f64(res["y"])[same], ref["y"][same]) <= tol_for(cfg)


def test_layer_is_deterministic():
    wl = to_device(generate(SMALL["qwen_zipf"], seed=3))
    a = run_layer(wl)["y"].clone()
    b = run_layer(wl)["y"]
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


EDGE = [dict(T=1), dict(T=3, E=64), dict(E=8, k=8), dict(T=257), dict(T=513, k=1),
        # I = I_shared = 128 (K a multiple of the 128-deep stage): the 32-row
        # tiled shape of decode plans, its down projection on 64-wide blocks,
        # with the one-launch permutation at 4, 8 and 16 mask words
        dict(T=1, I=128), dict(T=300, E=64, k=6, I=128), dict(T=700, E=32, k=2, I=128),
        dict(T=1000, E=256, k=8, I=128),
        # I = 2048: the down projection's 256-deep stages
        dict(T=40, E=16, k=4, I=2048)]


def edge_config(over):
    I = over.get("I", 64)
    return shrink(CONFIGS["qwen_decode"], D=128, E=over.get("E", 16), k=over.get("k", 4),
                  I=I, I_shared=I if I >= 128 else 64, T=over["T"] if "T" in over else 40)


@pytest.mark.parametrize("over", EDGE)
def test_layer_edge_shapes(over):
    cfg = edge_config(over)
    wl = to_device(generate(cfg, seed=4))
    ref = oracle_layer(wl)
    res = run_layer(wl, logits_in=torch.from_numpy(ref["logits"]).cuda())
    _check_routing(res, ref)
    assert rel_err(f64(res["y"]), ref["y"]) <= tol_for(cfg)


# The largest expert count and top-k the library takes (E = 1024, k = 32),
# through the one-launch permutation (T <= 1024) and the multi-block one
@pytest.mark.parametrize("T,policy", [(100, "auto"), (100, "lds"), (1100, "auto"), (1100, "lds")])
def test_layer_max_experts_and_k(T, policy):
    cfg = shrink(CONFIGS["qwen_decode"], T=T, D=128, E=1024, k=32, I=64, I_shared=64)
    print(f"[max E and k] T={T} policy={policy}", flush=True)
    wl = to_device(generate(cfg, seed=7))
    ref = oracle_layer(wl)
    res = run_layer(wl, policy, logits_in=torch.from_numpy(ref["logits"]).cuda())
    _check_routing(res, ref)
    assert rel_err(f64(res["y"]), ref["y"]) <= tol_for(cfg)


# A device router at T >= 512 with E not a multiple of 4: the LDS-tiled router
# stores four columns at a time, so such problems take the streamed router
@pytest.mark.parametrize("E", [10, 6])
def test_device_router_expert_count_not_multiple_of_four(E):
    cfg = shrink(CONFIGS["qwen_prefill"], T=512, D=256, E=E, k=2, I=64, I_shared=64, zipf=False)
    wl = to_device(generate(cfg, seed=12))
    ref = oracle_layer(wl)
    p = problem(cfg)
    logits = torch.empty((cfg.T, E), dtype=torch.float32, device="cuda")
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
    B.moe_route(p, wl.x, wl.wr, logits, False, idx, w)
    torch.cuda.synchronize()
    lr = ref["logits"].astype(np.float64)
    assert np.max(np.abs(f64(logits) - lr)) <= 1e-5 * max(1.0, float(np.max(np.abs(lr))))
    same = np.all(np.sort(idx.cpu().numpy(), 1) == np.sort(ref["idx"], 1), axis=1)
    assert same.mean() >= 0.99
    res = run_layer(wl)
    same = np.all(np.sort(res["topk_idx"].cpu().numpy(), 1) == np.sort(ref["idx"], 1), axis=1)
    assert same.mean() >= 0.99
    assert rel_err(f64(res["y"])[same], ref["y"][same]) <= tol_for(cfg)


# The router on 256-row tiles (from 4096 tokens with E a multiple of 256): a
# ragged last M-tile (T = 4099) and two or four K slices of partial sums.
ROUTER_TALL = [(512, 512), (1024, 256)]


def router_tall_config(D, E):
    return shrink(CONFIGS["qwen_prefill"], T=4099, D=D, E=E, k=4, I=64, I_shared=0, zipf=False)


@pytest.mark.parametrize("D,E", ROUTER_TALL)
def test_device_router_tall_tiles(D, E):
    cfg = router_tall_config(D, E)
    print(f"[router 256-row tiles] T={cfg.T} D={D} E={E}", flush=True)
    wl = to_device(generate(cfg, seed=13))
    ref = oracle_layer(wl)
    p = problem(cfg)
    logits = torch.empty((cfg.T, E), dtype=torch.float32, device="cuda")
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
    B.moe_route(p, wl.x, wl.wr, logits, False, idx, w)
    torch.cuda.synchronize()
    lr = ref["logits"].astype(np.float64)
    assert np.max(np.abs(f64(logits) - lr)) <= 1e-5 * max(1.0, float(np.max(np.abs(lr))))
    same = np.all(np.sort(idx.cpu().numpy(), 1) == np.sort(ref["idx"], 1), axis=1)
    assert same.mean() >= 0.99
    res = run_layer(wl)
    # the layer adds the K slices' partial sums (moe_route writes whole sums)
    assert np.max(np.abs(f64(res["logits"]) - lr)) <= 1e-5 * max(1.0, float(np.max(np.abs(lr))))
    same = np.all(np.sort(res["topk_idx"].cpu().numpy(), 1) == np.sort(ref["idx"], 1), axis=1)
    assert same.mean() >= 0.99
    assert rel_err(f64(res["y"])[same], ref["y"][same]) <= tol_for(cfg)


# 256-row tiles with skewed loads: hot experts with two to four tiles next to
# one-tile and empty experts, and one expert taking every token (16 tiles)
@pytest.mark.parametrize("T,k,skew", [(2000, 2, 0.15), (4096, 1, None)])
def test_layer_skewed_tall_tiles(T, k, skew):
    cfg = shrink(CONFIGS["qwen_prefill"], T=T, D=256, E=64, k=k, I=64, I_shared=64, zipf=False)
    print(f"[skewed 256-row tiles] T={T} k={k} skew={skew}", flush=True)
    wl = to_device(generate(cfg, seed=6))
    rng = np.random.default_rng(T)
    logits = rng.standard_normal((T, cfg.E)).astype(np.float32)
    if skew is None:
        logits[:, 0] += 100.0
    else:
        logits -= np.float32(skew) * np.arange(cfg.E, dtype=np.float32)
    ref = oracle_layer(wl, logits_in=logits)
    counts = np.asarray(ref["counts"])
    assert counts.max() > 256 and (skew is None or np.sum((counts > 0) & (counts <= 256)) > 8)
    res = run_layer(wl, "lds", logits_in=torch.from_numpy(logits).cuda())
    _check_routing(res, ref)
    assert rel_err(f64(res["y"]), ref["y"]) <= tol_for(cfg)


# fp32 plain-softmax weight: expf (2 ulp) of each term, a sum of E/64 terms per
# lane then 6 butterfly levels, and a divide: under 25 ulp (1.5e-6) for E <= 1024
PLAIN_W_RTOL = 3e-6


@pytest.mark.parametrize("policy", ["stream", "lds"])
@pytest.mark.parametrize("name", ["qwen_ragged", "ling_fp8", "big_groups_bf16"])
def test_layer_plain_softmax_gating(name, policy):
    """renormalize = 0: routing with oracle logits is bit-exact, the weights are
    the plain softmax probabilities, and the layer is within tolerance."""
    cfg = SMALL[name]
    wl = to_device(generate(cfg, seed=8))
    ref = oracle_layer(wl, renormalize=False)
    res = run_layer(wl, policy, logits_in=torch.from_numpy(ref["logits"]).cuda(), renormalize=False)
    _check_routing(res, ref, w_rtol=PLAIN_W_RTOL)
    assert np.all(ref["w"].sum(axis=1) < 1.0)
    assert rel_err(f64(res["y"]), ref["y"]) <= tol_for(cfg)


@pytest.mark.parametrize("T,E,k", [(300, 96, 6), (129, 1024, 32), (64, 8, 8)])
def test_moe_route_plain_softmax(T, E, k):
    l = np.random.default_rng(9).standard_normal((T, E)).astype(np.float32) * 2
    cfg = shrink(CONFIGS["qwen_decode"], T=T, D=128, E=E, k=k, I=64, I_shared=64)
    p = problem(cfg, renormalize=False)
    logits = torch.from_numpy(l).cuda()
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    B.moe_route(p, None, None, logits, True, idx, w)
    torch.cuda.synchronize()
    ri, rw = topk_softmax(l, k, renormalize=False)
    assert np.array_equal(idx.cpu().numpy(), ri)
    assert np.allclose(w.cpu().numpy(), rw, rtol=PLAIN_W_RTOL, atol=0)


@pytest.mark.parametrize("name,logits_given", [("qwen_decode_like", False), ("qwen_zipf", False),
                                                ("qwen_ragged", True), ("ling_fp8", False)])
def test_plan_query_matches_the_stages_run(name, logits_given):
    """moe_layer_plan describes what moe_layer runs: the stage record shows
    the tile-table stage exactly when the plan says the permutation is not one
    launch, and the router stage exactly when logits are not passed in."""
    cfg = SMALL[name]
    plan = B.moe_layer_plan(problem(cfg))
    wl = to_device(generate(cfg, seed=21))
    logits_in = None
    if logits_given:
        logits_in = torch.from_numpy(oracle_layer(wl)["logits"]).cuda()
    B.moe_timing_read()
    B.moe_timing_enable(True)
    try:
        run_layer(wl, logits_in=logits_in, want=())
        torch.cuda.synchronize()
    finally:
        B.moe_timing_enable(False)
    rec = B.moe_timing_read()
    assert rec["permute"][1] == 1 and rec["topk_softmax"][1] == 1
    assert rec["tile_table"][1] == (0 if plan["one_launch_permute"] else 1), (name, plan)
    assert rec["router_gemm"][1] == (0 if logits_given else 1), name


def test_stage_timing_mask():
    """Timing restricted to one stage records that stage only, and the output
    is the same as with timing off."""
    wl = to_device(generate(SMALL["qwen_zipf"], seed=3))
    ref = run_layer(wl)["y"].clone()
    names = [B.moe_stage_name(i) for i in range(B.moe_stage_count())]
    B.moe_timing_read()
    B.moe_timing_enable(True, stages=[names.index("ffn1_gate_up_act")])
    try:
        y = run_layer(wl)["y"]
        torch.cuda.synchronize()
    finally:
        B.moe_timing_enable(False)
    rec = B.moe_timing_read()
    assert rec["ffn1_gate_up_act"][1] == 1 and rec["ffn1_gate_up_act"][0] > 0
    assert all(n == 0 for k, (_, n) in rec.items() if k != "ffn1_gate_up_act")
    assert torch.equal(ref.view(torch.int16), y.view(torch.int16))
    B.moe_timing_enable(True)
    try:
        run_layer(wl)
        torch.cuda.synchronize()
    finally:
        B.moe_timing_enable(False)
    rec = B.moe_timing_read()
    assert rec["ffn1_gate_up_act"][1] == 1 and rec["ffn2_down"][1] == 1 and rec["combine"][1] == 1


def test_zero_tokens_enqueues_nothing():
    cfg = shrink(CONFIGS["qwen_decode"], T=0, D=128, E=8, k=2, I=64, I_shared=64)
    p = problem(cfg)
    args = B.layer_args(x=1, w_router=1, w13=1, w2=1, w13_shared=1, w2_shared=1, y=1)
    ws = torch.empty(max(B.moe_layer_workspace_size(p), 1), dtype=torch.uint8, device="cuda")
    B.moe_layer(p, args, ws, ws.numel())
    torch.cuda.synchronize()


# ------------------------------------------------------------------ entry points one by one
def test_moe_route_entry():
    cfg = SMALL["qwen_ragged"]
    wl = to_device(generate(cfg, seed=5))
    ref = oracle_layer(wl)
    p = problem(cfg)
    lg = torch.from_numpy(ref["logits"]).cuda()
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
    B.moe_route(p, None, None, lg, True, idx, w)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), ref["idx"])
    assert np.allclose(w.cpu().numpy(), ref["w"], rtol=1e-6, atol=0)


def test_moe_route_ties_and_signed_zero():
    T, E, k = 64, 40, 7
    rng = np.random.default_rng(0)
    l = rng.standard_normal((T, E)).astype(np.float32)
    l[:, 3] = l[:, 1]
    l[::2, 5] = l[::2, 0]
    l[1::3, 2], l[1::3, 6] = 0.0, -0.0
    l[7, :] = 2.5
    p = B.make_problem(T, 64, E, k, 64)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    B.moe_route(p, None, None, torch.from_numpy(l).cuda(), True, idx, w)
    torch.cuda.synchronize()
    ri, rw = topk_softmax(l, k)
    assert np.array_equal(idx.cpu().numpy(), ri)
    assert np.allclose(w.cpu().numpy(), rw, rtol=1e-6, atol=0)


@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (255, 16, 4), (256, 16, 4), (300, 64, 4), (1000, 512, 10),
                                   (1024, 1024, 8), (1025, 64, 2), (4099, 256, 8), (600, 1024, 32)])
def test_moe_permute_entry(T, E, k):
    rng = np.random.default_rng(T + E)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    p = B.make_problem(T, 64, E, k, 64)
    d = {n: torch.empty(s, dtype=torch.int32, device="cuda") for n, s in
         (("counts", E), ("offsets", E + 1), ("row_token", T * k), ("row_of_slot", T * k))}
    n = B.moe_permute_workspace_size(p)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    B.moe_permute(p, torch.from_numpy(idx).cuda(), d["counts"], d["offsets"], d["row_token"],
                  d["row_of_slot"], ws, n)
    torch.cuda.synchronize()
    ref = dict(zip(("counts", "offsets", "row_token", "row_of_slot"), permute(idx, E)))
    for name in ref:
        assert np.array_equal(d[name].cpu().numpy(), ref[name]), name


@pytest.mark.parametrize("T,E,k,D,dt,bad", [(300, 64, 4, 256, "bf16", False), (1100, 16, 3, 192, "f32", False),
                                             (4099, 256, 8, 512, "bf16", False), (700, 32, 2, 128, "bf16", True)])
def test_moe_permute_materialised_gather(T, E, k, D, dt, bad):
    """x_perm[r] = x[row_token[r]] bit for bit; with out-of-range ids the rows
    past offsets[E] are left as they were."""
    rng = np.random.default_rng(T + D)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    if bad:
        idx[::5, 0] = E + 3
    p = B.make_problem(T, D, E, k, 64, act_dtype=dt, w_dtype=dt)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    x = torch.randn(T, D, dtype=torch.float32).to(tdt).cuda()
    xp = torch.full((T * k, D), 7.0, dtype=tdt, device="cuda")
    d = {n: torch.empty(sz, dtype=torch.int32, device="cuda") for n, sz in
         (("counts", E), ("offsets", E + 1), ("row_token", T * k), ("row_of_slot", T * k))}
    n = B.moe_permute_workspace_size(p)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    B.moe_permute(p, torch.from_numpy(idx).cuda(), d["counts"], d["offsets"], d["row_token"],
                  d["row_of_slot"], ws, n, x=x, x_perm=xp)
    torch.cuda.synchronize()
    valid = np.where(idx < E, idx, 0)
    if bad:   # the oracle's permutation of the valid assignments only
        flat = idx.reshape(-1)
        keep = np.flatnonzero(flat < E)
        order = keep[np.argsort(flat[keep], kind="stable")]
        row_token = order // k
    else:
        row_token = permute(valid, E)[2]
    filled = len(row_token)
    xh, xph = x.cpu(), xp.cpu()
    assert torch.equal(xph[:filled].view(torch.int16 if dt == "bf16" else torch.int32),
                       xh[torch.from_numpy(row_token.astype(np.int64))].view(torch.int16 if dt == "bf16"
                                                                              else torch.int32))
    assert torch.all(xph[filled:] == 7.0)


def test_grouped_ffn_on_materialised_rows_matches_gathered():
    """The grouped FFN on x_perm (row_token = NULL) gives the gathered path's
    output bit for bit, and both match the oracle."""
    cfg = SMALL["qwen_ragged"]
    wl = to_device(generate(cfg, seed=13))
    ref = oracle_layer(wl, keep=True)
    T, k, D, E = cfg.T, cfg.k, cfg.D, cfg.E
    p = problem(cfg)
    d = {n: torch.empty(sz, dtype=torch.int32, device="cuda") for n, sz in
         (("counts", E), ("offsets", E + 1), ("row_token", T * k), ("row_of_slot", T * k))}
    xp = torch.empty((T * k, D), dtype=torch.bfloat16, device="cuda")
    n = B.moe_permute_workspace_size(p)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    B.moe_permute(p, torch.from_numpy(np.asarray(ref["idx"])).cuda(), d["counts"], d["offsets"],
                  d["row_token"], d["row_of_slot"], ws, n, x=wl.x, x_perm=xp)
    outs = []
    for a, rt in ((wl.x, d["row_token"]), (xp, None)):
        h = torch.empty((T * k, cfg.I), dtype=torch.bfloat16, device="cuda")
        out = torch.empty((T * k, D), dtype=torch.bfloat16, device="cuda")
        nf = B.moe_grouped_ffn_workspace_size(p, E, T * k)
        wsf = torch.empty(max(nf, 1), dtype=torch.uint8, device="cuda")
        B.moe_grouped_ffn(p, E, T * k, a, rt, d["offsets"], wl.w13, wl.s13, wl.w2, wl.s2, h, out, wsf, nf)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    assert rel_err(f64(outs[1]), ref["o_perm"]) <= tol_for(cfg)


def test_measurement_probes_run():
    """The HBM-read and MFMA probes the benchmark reports run and count FLOPs."""
    buf = torch.randint(0, 255, (64 << 20,), dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    B.moe_probe_hbm_read(buf, buf.numel(), sink)
    ops = torch.randn(65536, dtype=torch.float32)          # 64 KiB of operands for either type
    nsink = B.moe_probe_mfma_sink_floats()
    fs = torch.empty(nsink, dtype=torch.float32, device="cuda")
    for dt, o in (("bf16", ops[:32768].to(torch.bfloat16)), ("fp8", ops.to(torch.float8_e4m3fn))):
        flop = B.moe_probe_mfma(dt, o.view(torch.uint8).cuda(), 4, fs)
        torch.cuda.synchronize()
        assert flop > 0 and torch.isfinite(fs).all()


def test_moe_combine_reproduces_gathered_rows():
    """o_perm := x gathered through the permutation gives y = x * sum(w) = x."""
    T, E, k, D = 200, 16, 4, 256
    rng = np.random.default_rng(1)
    l = rng.standard_normal((T, E)).astype(np.float32)
    idx, w = topk_softmax(l, k)
    _, _, row_token, row_of_slot = permute(idx, E)
    x = torch.randn(T, D, dtype=torch.float32)
    o = x[torch.from_numpy(row_token.astype(np.int64))].contiguous()
    p = B.make_problem(T, D, E, k, 64, act_dtype="f32", w_dtype="f32")
    y = torch.empty(T, D, device="cuda")
    B.moe_combine(p, o.cuda(), torch.from_numpy(row_of_slot).cuda(), torch.from_numpy(w).cuda(),
                  None, y)
    torch.cuda.synchronize()
    assert rel_err(y.cpu().numpy(), x.numpy()) < 1e-6


def test_moe_combine_drops_rows_out_of_range():
    """Assignments whose row is negative or not below T*k add nothing."""
    T, k, D = 64, 3, 128
    rng = np.random.default_rng(2)
    o = torch.randn(T * k, D, dtype=torch.float32)
    rows = rng.permutation(T * k).astype(np.int32).reshape(T, k)
    rows[::3, 0] = -1
    rows[1::3, 1] = T * k
    rows[2::5, 2] = np.iinfo(np.int32).max
    w = rng.random((T, k)).astype(np.float32)
    sh = torch.randn(T, D, dtype=torch.float32)
    p = B.make_problem(T, D, 8, k, 64, act_dtype="f32", w_dtype="f32")
    y = torch.empty(T, D, device="cuda")
    B.moe_combine(p, o.cuda(), torch.from_numpy(rows).cuda(), torch.from_numpy(w).cuda(), sh.cuda(), y)
    torch.cuda.synchronize()
    on = torch.from_numpy((rows >= 0) & (rows < T * k))
    idx = torch.from_numpy(np.clip(rows, 0, T * k - 1).astype(np.int64))
    ref = (o.double()[idx] * (torch.from_numpy(w).double() * on)[..., None]).sum(1) + sh.double()
    assert torch.allclose(y.cpu().double(), ref, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("policy", ["stream", "lds", "auto"])
@pytest.mark.parametrize("name", ["qwen_ragged", "ling_fp8", "gemma_like", "ling_decode_like",
                                  "qwen_decode_deep"])
def test_moe_grouped_ffn_entry(name, policy):
    """Grouped FFN alone on permuted rows, and the shared branch as one group."""
    cfg = SMALL[name]
    wl = to_device(generate(cfg, seed=6))
    ref = oracle_layer(wl, keep=True)
    rows = cfg.T * cfg.k
    p = problem(cfg, policy)
    h = torch.empty((rows, cfg.I), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((rows, cfg.D), dtype=torch.bfloat16, device="cuda")
    n = B.moe_grouped_ffn_workspace_size(p, cfg.E, rows)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    B.moe_grouped_ffn(p, cfg.E, rows, wl.x, torch.from_numpy(ref["row_token"]).cuda(),
                      torch.from_numpy(ref["offsets"]).cuda(), wl.w13, wl.s13, wl.w2, wl.s2, h, out,
                      ws, n)
    torch.cuda.synchronize()
    tol = tol_for(cfg)
    assert rel_err(f64(h), ref["h_perm"]) <= tol
    assert rel_err(f64(out), ref["o_perm"]) <= tol
    # the shared branch: one group over all tokens, identity rows
    ps = B.make_problem(cfg.T, cfg.D, 1, 1, cfg.I_shared, 0, cfg.act_shared, cfg.act_shared,
                        cfg.act_dtype, cfg.shared_w_dtype, cfg.shared_w_dtype, policy)
    hs = torch.empty((cfg.T, cfg.I_shared), dtype=torch.bfloat16, device="cuda")
    os_ = torch.empty((cfg.T, cfg.D), dtype=torch.bfloat16, device="cuda")
    n = B.moe_grouped_ffn_workspace_size(ps, 1, cfg.T)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    B.moe_grouped_ffn(ps, 1, cfg.T, wl.x, None, torch.tensor([0, cfg.T], dtype=torch.int32).cuda(),
                      wl.w13s, wl.s13s, wl.w2s, wl.s2s, hs, os_, ws, n)
    torch.cuda.synchronize()
    assert rel_err(f64(os_), ref["shared_out"]) <= tol


# ------------------------------------------------------------------ full-size configs
FULL = ["qwen_decode", "gemma", "ling_decode", "qwen_prefill", "ling_prefill"]


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """Largest over tokens of max|got - ref| / max|ref| within the token's row,
    so an error confined to rows of small magnitude is not hidden by the
    tensor-wide normalisation."""
    den = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return float(np.max(np.abs(got - ref).max(axis=1) / den))


@pytest.mark.parametrize("name", FULL)
def test_full_size_layer(name):
    """Every element of y at the benchmark sizes, against the whole-layer oracle."""
    cfg = CONFIGS[name]
    print(f"[full-size] {name}: generating on GPU", flush=True)
    wl = generate(cfg, seed=0, weight_device="cuda")
    to_device(wl)
    x, wr, expert, shared = oracle_inputs(wl)
    logits_ref = router_logits(x, wr)
    print(f"[full-size] {name}: running moe_layer with oracle logits", flush=True)
    res = run_layer(wl, logits_in=torch.from_numpy(logits_ref).cuda())
    y = f64(res["y"])
    print(f"[full-size] {name}: oracle, whole layer", flush=True)
    ref = layer(x, wr, cfg.k, expert, shared, cfg.act, cfg.act_shared, logits_in=logits_ref)
    _check_routing(res, ref)
    err, rerr = rel_err(y, ref["y"]), row_rel_err(y, ref["y"])
    print(f"[full-size] {name}: rel err {err:.3e} (worst row {rerr:.3e})", flush=True)
    assert err <= tol_for(cfg)
    assert rerr <= 3 * tol_for(cfg)
    # fully on device: logits within tolerance; top-k sets may flip only on
    # near-ties; tokens whose set agrees match the oracle's y
    res2 = run_layer(wl)
    lg = f64(res2["logits"])
    assert np.max(np.abs(lg - logits_ref)) <= 1e-5 * max(1.0, float(np.max(np.abs(logits_ref))))
    same = np.all(np.sort(res2["topk_idx"].cpu().numpy(), 1) == np.sort(ref["idx"], 1), axis=1)
    print(f"[full-size] {name}: tokens whose top-k set differs: {int((~same).sum())}", flush=True)
    assert same.mean() >= 0.999
    assert rel_err(f64(res2["y"])[same], ref["y"][same]) <= tol_for(cfg)
    del wl, res, res2, ref, y
    torch.cuda.empty_cache()


def test_layer_past_2e31_elements():
    """A layer whose permuted expert rows o [T*k, D] pass 2^31 elements (64-bit
    offsets everywhere but the tiled GEMM's per-operand 32-bit byte offsets),
    against the oracle on every token with a row past element 2^31 that a
    sample draws, plus random tokens and the first and last."""
    cfg = shrink(CONFIGS["ling_prefill"], T=36000, D=8192, E=16, k=8, I=256, I_shared=256)
    assert cfg.T * cfg.k * cfg.D > 2 ** 31
    print("[large-T] generating", flush=True)
    wl = generate(cfg, seed=5, weight_device="cuda")
    to_device(wl)
    x, wr, expert, shared = oracle_inputs(wl)
    logits = router_logits(x, wr)
    idx, w = topk_softmax(logits, cfg.k)
    _, _, row_token, _ = permute(idx, cfg.E)
    print("[large-T] running moe_layer with oracle logits", flush=True)
    res = run_layer(wl, logits_in=torch.from_numpy(logits).cuda(), want=("topk_idx_out", "row_token_out"))
    assert np.array_equal(res["topk_idx"].cpu().numpy(), idx)
    assert np.array_equal(res["row_token"].cpu().numpy(), row_token)
    late = np.unique(row_token[2 ** 31 // cfg.D:])     # tokens with a row past element 2^31
    rng = np.random.default_rng(0)
    toks = sorted(set(rng.choice(late, 48, replace=False).tolist())
                  | set(rng.choice(cfg.T, 16, replace=False).tolist()) | {0, cfg.T - 1})
    print(f"[large-T] oracle on {len(toks)} tokens", flush=True)
    ref = layer_tokens(toks, x, idx, w, expert, shared, cfg.act, cfg.act_shared)
    err = rel_err(f64(res["y"])[toks], ref)
    print(f"[large-T] rel err {err:.3e}", flush=True)
    assert err <= tol_for(cfg)
    del wl, res
    torch.cuda.empty_cache()
