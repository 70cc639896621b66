"""The C-ABI library builds, loads and exports every declared entry point, and
its host-side validation returns the documented status codes (CPU only: none of
these calls reaches a kernel launch)."""
import ctypes
import os
import re
import subprocess

import pytest

from sparse_mixture_experts_moe_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from sparse_mixture_experts_moe_amd.build import build
        build(verbose=False)
    return B.lib()


def declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:moe_status_t|const char\*|int32_t|size_t)\s+(moe_\w+)\s*\(", txt, re.M)))


def test_header_declares_the_entry_points():
    names = declared()
    for n in ("moe_route", "moe_permute", "moe_grouped_ffn", "moe_combine", "moe_layer",
              "moe_layer_workspace_size", "moe_status_string"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT\s+(moe_\w+)", out))
    for n in declared():
        assert n in exported, n
        assert hasattr(lib, n)
    assert set(B.exported_symbols()) == set(declared())


def test_status_strings(lib):
    for st in range(7):
        assert B.status_string(st)
    assert B.status_string(4) == "unsupported combination"


def _ok_problem(**over):
    p = B.make_problem(64, 256, 8, 2, 128, 0, act_dtype="f32", w_dtype="f32")
    for k, v in over.items():
        setattr(p, k, v)
    return p


@pytest.mark.parametrize("over,status", [
    (dict(D=100), B.MOE_ERR_SHAPE), (dict(I=96), B.MOE_ERR_SHAPE), (dict(E=0), B.MOE_ERR_SHAPE),
    (dict(E=2000), B.MOE_ERR_SHAPE), (dict(k=9), B.MOE_ERR_SHAPE), (dict(k=0), B.MOE_ERR_SHAPE),
    (dict(k=33, E=64), B.MOE_ERR_SHAPE), (dict(T=-1), B.MOE_ERR_SHAPE),
    (dict(I_shared=32), B.MOE_ERR_SHAPE), (dict(T=2 ** 30), B.MOE_ERR_SHAPE),
    (dict(act=7), B.MOE_ERR_DTYPE), (dict(w_dtype=9), B.MOE_ERR_DTYPE),
    (dict(tile_policy=5), B.MOE_ERR_DTYPE),
    (dict(w_dtype=B.MOE_BF16), B.MOE_ERR_UNSUPPORTED),              # f32 act x bf16 weights
    (dict(act_dtype=B.MOE_FP8_E4M3FN), B.MOE_ERR_UNSUPPORTED),
    (dict(renormalize=2), B.MOE_ERR_UNSUPPORTED), (dict(act_quant=2), B.MOE_ERR_UNSUPPORTED),
    (dict(act_quant=3), B.MOE_ERR_UNSUPPORTED), (dict(act_quant=-1), B.MOE_ERR_UNSUPPORTED),
    (dict(act_dtype=B.MOE_MXFP4_E2M1), B.MOE_ERR_DTYPE),               # weights-only format
    (dict(act_quant=1), B.MOE_ERR_UNSUPPORTED),                       # fp32 layer: no fp8 path
    (dict(renormalize=0), B.MOE_OK),
    (dict(combine=3), B.MOE_ERR_UNSUPPORTED), (dict(combine=-1), B.MOE_ERR_UNSUPPORTED),
    (dict(T=2 ** 22), B.MOE_OK),                                      # (T*k + T) * D past 2^31
    (dict(combine=B.MOE_COMBINE_SEPARATE), B.MOE_OK), (dict(combine=B.MOE_COMBINE_FUSED), B.MOE_OK),
])
def test_validation_codes(lib, over, status):
    p = _ok_problem(**over)
    n = ctypes.c_size_t(0)
    assert lib.moe_layer_workspace_size(ctypes.byref(p), ctypes.byref(n)) == status


def _fp8_problem(**over):
    p = B.make_problem(64, 256, 8, 2, 128, 128, act_dtype="bf16", w_dtype="fp8",
                       act_quant=B.MOE_ACT_QUANT_FP8_ROW)
    for k, v in over.items():
        setattr(p, k, v)
    return p


@pytest.mark.parametrize("over,status", [
    (dict(), B.MOE_OK),
    (dict(w_dtype=B.MOE_BF16, shared_w_dtype=B.MOE_BF16), B.MOE_ERR_UNSUPPORTED),  # needs fp8 weights
    (dict(shared_w_dtype=B.MOE_BF16), B.MOE_ERR_UNSUPPORTED),
    (dict(tile_policy=B.MOE_TILE_STREAM), B.MOE_ERR_UNSUPPORTED),
    (dict(D=192), B.MOE_ERR_UNSUPPORTED), (dict(I=64), B.MOE_ERR_UNSUPPORTED),   # K multiple of 128
    (dict(I_shared=0), B.MOE_OK), (dict(D=32768), B.MOE_ERR_UNSUPPORTED),
    (dict(T=200000, D=8192), B.MOE_OK),         # past 2^31 elements, x under 4 GiB
    (dict(T=300000, D=8192), B.MOE_ERR_SHAPE),  # x past 4 GiB: the tiled GEMM (the only fp8 x fp8 one) cannot
])
def test_act_quant_validation(lib, over, status):
    p = _fp8_problem(**over)
    n = ctypes.c_size_t(0)
    assert lib.moe_layer_workspace_size(ctypes.byref(p), ctypes.byref(n)) == status
    if status == B.MOE_OK:
        p0 = _fp8_problem(act_quant=0, **over)
        assert n.value > B.moe_layer_workspace_size(p0)    # fp8 copies of x and h live there


def _mx_problem(**over):
    p = B.make_problem(64, 256, 8, 2, 128, 128, act_dtype="bf16", w_dtype="mxfp4",
                       act_quant=B.MOE_ACT_QUANT_MXFP8)
    for k, v in over.items():
        setattr(p, k, v)
    return p


@pytest.mark.parametrize("over,status", [
    (dict(), B.MOE_OK), (dict(I_shared=0), B.MOE_OK),
    (dict(act_quant=B.MOE_ACT_QUANT_NONE), B.MOE_ERR_UNSUPPORTED),     # MXFP4 needs MXFP8 activations
    (dict(act_quant=B.MOE_ACT_QUANT_FP8_ROW), B.MOE_ERR_UNSUPPORTED),
    (dict(w_dtype=B.MOE_FP8_E4M3FN), B.MOE_ERR_UNSUPPORTED),            # MXFP8 needs MXFP4 weights
    (dict(shared_w_dtype=B.MOE_FP8_E4M3FN), B.MOE_ERR_UNSUPPORTED),
    (dict(shared_w_dtype=B.MOE_BF16, I_shared=0), B.MOE_OK),            # no shared branch: unused
    (dict(tile_policy=B.MOE_TILE_STREAM), B.MOE_ERR_UNSUPPORTED),
    (dict(D=192), B.MOE_ERR_UNSUPPORTED), (dict(I=64), B.MOE_ERR_UNSUPPORTED),
    (dict(I_shared=64), B.MOE_ERR_UNSUPPORTED), (dict(D=32768), B.MOE_ERR_UNSUPPORTED),
    (dict(act_dtype=B.MOE_F32), B.MOE_ERR_UNSUPPORTED),
])
def test_mx_validation(lib, over, status):
    p = _mx_problem(**over)
    n = ctypes.c_size_t(0)
    assert lib.moe_layer_workspace_size(ctypes.byref(p), ctypes.byref(n)) == status
    assert lib.moe_grouped_ffn_workspace_size(ctypes.byref(p), 8, 128, ctypes.byref(n)) == status


def test_mx_workspace_holds_the_block_scales(lib):
    """The MXFP8 copies of x, h and h_shared take one byte per element plus
    one scale byte per 32 elements."""
    p, p0 = _mx_problem(T=1000), _mx_problem(T=1000)
    p0.act_quant, p0.w_dtype, p0.shared_w_dtype = 0, B.MOE_BF16, B.MOE_BF16
    T, D, k, I, Is = 1000, 256, 2, 128, 128
    extra = B.moe_layer_workspace_size(p) - B.moe_layer_workspace_size(p0)
    want = (T * D + T * k * I + T * Is) * (1 + 1 / 32)
    assert want <= extra <= want + 6 * 256


def test_quantize_rows_mx_validation(lib):
    fake = 4096
    f = lib.moe_quantize_rows_mx
    assert f(fake, 4, 64, 64, fake, fake, None) == B.MOE_ERR_SHAPE        # cols % 128
    assert f(fake, 4, 256, 128, fake, fake, None) == B.MOE_ERR_SHAPE      # lda < cols
    assert f(fake, 4, 128, 132, fake, fake, None) == B.MOE_ERR_SHAPE      # lda % 8
    assert f(fake, 4, 1 << 15, 1 << 15, fake, fake, None) == B.MOE_ERR_SHAPE
    assert f(fake, -1, 128, 128, fake, fake, None) == B.MOE_ERR_SHAPE
    assert f(fake + 8, 4, 128, 128, fake, fake, None) == B.MOE_ERR_SHAPE   # a 16-byte aligned
    assert f(None, 4, 128, 128, fake, fake, None) == B.MOE_ERR_NULL
    assert f(fake, 4, 128, 128, fake, None, None) == B.MOE_ERR_NULL
    assert f(None, 0, 128, 128, None, None, None) == B.MOE_OK


def _sub_problem(**over):
    p = B.make_problem(64, 1024, 8, 2, 512, 512, act_dtype="bf16", w_dtype="fp8",
                       act_quant=B.MOE_ACT_QUANT_FP8_SUB)
    for k, v in over.items():
        setattr(p, k, v)
    return p


@pytest.mark.parametrize("over,status", [
    (dict(), B.MOE_OK), (dict(I_shared=0), B.MOE_OK),
    (dict(D=768), B.MOE_ERR_UNSUPPORTED), (dict(I=256), B.MOE_ERR_UNSUPPORTED),   # K multiple of 512
    (dict(I_shared=1536), B.MOE_OK), (dict(I_shared=640), B.MOE_ERR_UNSUPPORTED),
    (dict(w_dtype=B.MOE_BF16, shared_w_dtype=B.MOE_BF16), B.MOE_ERR_UNSUPPORTED),
    (dict(tile_policy=B.MOE_TILE_STREAM), B.MOE_ERR_UNSUPPORTED),
    (dict(act_quant=4), B.MOE_ERR_UNSUPPORTED),
])
def test_subchannel_validation(lib, over, status):
    p = _sub_problem(**over)
    n = ctypes.c_size_t(0)
    assert lib.moe_layer_workspace_size(ctypes.byref(p), ctypes.byref(n)) == status
    assert lib.moe_grouped_ffn_workspace_size(ctypes.byref(p), 8, 128, ctypes.byref(n)) == status


def test_subchannel_workspace_holds_the_slice_scales(lib):
    """The fp8 copies of x, h and h_shared take one byte per element plus one
    fp32 scale per 512 elements."""
    p, p0 = _sub_problem(T=1000), _sub_problem(T=1000)
    p0.act_quant = 0
    T, D, k, I, Is = 1000, 1024, 2, 512, 512
    extra = B.moe_layer_workspace_size(p) - B.moe_layer_workspace_size(p0)
    want = (T * D + T * k * I + T * Is) * (1 + 4 / 512)
    assert want <= extra <= want + 6 * 256


def test_quantize_subchannel_validation(lib):
    fake = 4096
    f = lib.moe_quantize_subchannel
    assert f(fake, 4, 256, 256, fake, fake, None) == B.MOE_ERR_SHAPE      # cols % 512
    assert f(fake, 4, 1024, 512, fake, fake, None) == B.MOE_ERR_SHAPE     # lda < cols
    assert f(fake, 4, 512, 516, fake, fake, None) == B.MOE_ERR_SHAPE      # lda % 8
    assert f(fake, 4, 1 << 15, 1 << 15, fake, fake, None) == B.MOE_ERR_SHAPE
    assert f(fake, -1, 512, 512, fake, fake, None) == B.MOE_ERR_SHAPE
    assert f(fake + 8, 4, 512, 512, fake, fake, None) == B.MOE_ERR_SHAPE   # a 16-byte aligned
    assert f(None, 4, 512, 512, fake, fake, None) == B.MOE_ERR_NULL
    assert f(fake, 4, 512, 512, fake, None, None) == B.MOE_ERR_NULL
    assert f(None, 0, 512, 512, None, None, None) == B.MOE_OK


def test_quantize_rows_validation(lib):
    fake = 4096
    assert lib.moe_quantize_rows(fake, 4, 12, 16, fake, fake, None) == B.MOE_ERR_SHAPE   # cols % 8
    assert lib.moe_quantize_rows(fake, 4, 16, 8, fake, fake, None) == B.MOE_ERR_SHAPE    # lda < cols
    assert lib.moe_quantize_rows(fake, 4, 16, 20, fake, fake, None) == B.MOE_ERR_SHAPE   # lda % 8
    assert lib.moe_quantize_rows(fake, 4, 1 << 15, 1 << 15, fake, fake, None) == B.MOE_ERR_SHAPE
    assert lib.moe_quantize_rows(fake, -1, 16, 16, fake, fake, None) == B.MOE_ERR_SHAPE
    assert lib.moe_quantize_rows(None, 4, 16, 16, fake, fake, None) == B.MOE_ERR_NULL
    assert lib.moe_quantize_rows(None, 0, 16, 16, None, None, None) == B.MOE_OK


def test_null_and_workspace_errors(lib):
    p = _ok_problem()
    n = ctypes.c_size_t(0)
    assert lib.moe_layer_workspace_size(None, ctypes.byref(n)) == B.MOE_ERR_NULL
    assert lib.moe_layer_workspace_size(ctypes.byref(p), None) == B.MOE_ERR_NULL
    need = B.moe_layer_workspace_size(p)
    assert need > 0
    fake = 4096  # never dereferenced: validation fails before anything is enqueued
    args = B.layer_args(x=fake, w_router=fake, w13=fake, w2=fake, y=fake)
    assert lib.moe_layer(ctypes.byref(p), ctypes.byref(args), fake, need - 1, None) == B.MOE_ERR_WORKSPACE
    assert lib.moe_layer(ctypes.byref(p), ctypes.byref(args), None, need, None) == B.MOE_ERR_NULL
    bad = B.layer_args(x=fake, w13=fake, w2=fake, y=fake)          # no router and no logits
    assert lib.moe_layer(ctypes.byref(p), ctypes.byref(bad), fake, need, None) == B.MOE_ERR_NULL
    ps = B.make_problem(64, 256, 8, 2, 128, 64, act_dtype="bf16", w_dtype="fp8")
    need = B.moe_layer_workspace_size(ps)
    args = B.layer_args(x=fake, w_router=fake, w13=fake, w2=fake, y=fake)   # fp8 without scales
    assert lib.moe_layer(ctypes.byref(ps), ctypes.byref(args), fake, need, None) == B.MOE_ERR_NULL
    assert lib.moe_route(ctypes.byref(p), fake, fake, None, 0, fake, fake, None) == B.MOE_ERR_NULL
    assert lib.moe_combine(ctypes.byref(p), None, fake, fake, None, fake, None) == B.MOE_ERR_NULL
    assert lib.moe_permute(ctypes.byref(p), fake, fake, fake, fake, fake, None, None, None, 0,
                           None) == B.MOE_ERR_NULL
    nperm = B.moe_permute_workspace_size(p)
    # x and x_perm go together, 16-byte aligned
    assert lib.moe_permute(ctypes.byref(p), fake, fake, fake, fake, fake, fake, None, fake, nperm,
                           None) == B.MOE_ERR_NULL
    assert lib.moe_permute(ctypes.byref(p), fake, fake, fake, fake, fake, None, fake, fake, nperm,
                           None) == B.MOE_ERR_NULL
    assert lib.moe_permute(ctypes.byref(p), fake, fake, fake, fake, fake, fake + 8, fake, fake, nperm,
                           None) == B.MOE_ERR_SHAPE
    # measurement probes: sizes and dtypes are checked before any launch
    flop = ctypes.c_double(0)
    assert lib.moe_probe_hbm_read(fake, 100, fake, None) == B.MOE_ERR_SHAPE
    assert lib.moe_probe_hbm_read(None, 1 << 20, fake, None) == B.MOE_ERR_NULL
    assert lib.moe_probe_mfma(B.MOE_F32, fake, 10, fake, ctypes.byref(flop), None) == B.MOE_ERR_DTYPE
    assert lib.moe_probe_mfma(B.MOE_BF16, fake, 0, fake, ctypes.byref(flop), None) == B.MOE_ERR_SHAPE
    assert lib.moe_probe_mfma_sink_floats() > 0
    assert lib.moe_grouped_ffn(ctypes.byref(p), 0, 10, fake, None, fake, fake, None, fake, None,
                               fake, fake, fake, 1 << 20, None) == B.MOE_ERR_SHAPE
    assert lib.moe_debug_fp8_to_bf16(fake, fake, 7, None) == B.MOE_ERR_SHAPE
    assert lib.moe_debug_f32_to_fp8(fake, fake, 7, None) == B.MOE_ERR_SHAPE
    assert lib.moe_debug_f32_to_fp8(None, fake, 8, None) == B.MOE_ERR_NULL


def test_grouped_ffn_rows_bound(lib):
    """rows_upper_bound * max(D, I) must stay below 2^31, whatever T and k say."""
    p = B.make_problem(64, 8192, 8, 2, 2048, 0)
    n = ctypes.c_size_t(0)
    ok = (1 << 31) // 8192 - 1
    assert lib.moe_grouped_ffn_workspace_size(ctypes.byref(p), 8, ok, ctypes.byref(n)) == B.MOE_OK
    assert lib.moe_grouped_ffn_workspace_size(ctypes.byref(p), 8, ok + 1, ctypes.byref(n)) == B.MOE_ERR_SHAPE
    fake = 4096
    assert lib.moe_grouped_ffn(ctypes.byref(p), 8, ok + 1, fake, None, fake, fake, None, fake, None,
                               fake, fake, fake, 1 << 40, None) == B.MOE_ERR_SHAPE
    q = B.make_problem(64, 256, 8, 2, 16384, 0)
    assert lib.moe_grouped_ffn_workspace_size(ctypes.byref(q), 8, (1 << 31) // 16384,
                                              ctypes.byref(n)) == B.MOE_ERR_SHAPE


def test_zero_tokens_is_ok_and_launches_nothing(lib):
    p = _ok_problem(T=0)
    need = B.moe_layer_workspace_size(p)
    fake = 4096
    args = B.layer_args(x=fake, w_router=fake, w13=fake, w2=fake, y=fake)
    assert lib.moe_layer(ctypes.byref(p), ctypes.byref(args), fake, need, None) == B.MOE_OK
    assert lib.moe_route(ctypes.byref(p), fake, fake, fake, 0, fake, fake, None) == B.MOE_OK


def test_workspace_size_grows_with_tokens(lib):
    a = B.moe_layer_workspace_size(B.make_problem(64, 4096, 512, 10, 1024, 1024))
    b = B.moe_layer_workspace_size(B.make_problem(8192, 4096, 512, 10, 1024, 1024))
    assert b > a > 0
    # h and o of every routed and shared row, in bf16
    assert b >= (8192 * 10 + 8192) * (4096 + 1024) * 2
