"""ctypes binding of the C ABI in include/moe.h (argument marshalling only).

Every entry point has the C name and argument order.  Tensor arguments accept a
torch tensor (its data_ptr() is passed), a plain integer device address, or
None for a NULL pointer.  `stream` defaults to torch's current stream.  A
non-OK status raises MoeError.  Nothing here computes any part of the layer:
if the HIP library is not built, loading fails with MoeLibraryMissing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")

MOE_F32, MOE_BF16, MOE_FP8_E4M3FN, MOE_MXFP4_E2M1 = 0, 1, 2, 3
MOE_ACT_SILU, MOE_ACT_GELU_TANH = 0, 1
MOE_TILE_AUTO, MOE_TILE_STREAM, MOE_TILE_LDS = 0, 1, 2
MOE_ACT_QUANT_NONE, MOE_ACT_QUANT_FP8_ROW, MOE_ACT_QUANT_MXFP8, MOE_ACT_QUANT_FP8_SUB = 0, 1, 2, 3
MOE_SUBCHANNEL = 512
MOE_COMBINE_AUTO, MOE_COMBINE_SEPARATE, MOE_COMBINE_FUSED = 0, 1, 2
MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE = 0, 1, 2, 3
MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_LAUNCH = 4, 5, 6

DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3FN, "mxfp4": MOE_MXFP4_E2M1}
ACTS = {"silu": MOE_ACT_SILU, "gelu_tanh": MOE_ACT_GELU_TANH}
POLICIES = {"auto": MOE_TILE_AUTO, "stream": MOE_TILE_STREAM, "lds": MOE_TILE_LDS}
COMBINES = {"auto": MOE_COMBINE_AUTO, "separate": MOE_COMBINE_SEPARATE, "fused": MOE_COMBINE_FUSED}
# moe_plan_shape_t codes, by name
PLAN_SHAPES = ("stream16", "stream32", "stream64", "tiled256x256", "tiled128x512", "tiled128x256",
               "tiled32x128", "tiled64x256", "tiled32x64")


class MoeLibraryMissing(RuntimeError):
    pass


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class MoeProblem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "T", "D", "E", "k", "I", "I_shared", "act", "act_shared", "renormalize",
        "act_dtype", "w_dtype", "shared_w_dtype", "tile_policy", "act_quant", "combine")]


_vp = ctypes.c_void_p


class MoePlan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("router", "router_slices", "gate_up", "down",
                                              "one_launch_permute")]


class MoeLayerArgs(ctypes.Structure):
    _fields_ = [(n, _vp) for n in (
        "x", "w_router", "logits_in", "w13", "s13", "w2", "s2", "w13_shared", "s13_shared",
        "w2_shared", "s2_shared", "y", "logits_out", "topk_idx_out", "topk_w_out",
        "counts_out", "offsets_out", "row_token_out", "row_of_slot_out")]


_LIB = None
_SIG = {
    "moe_route": [ctypes.POINTER(MoeProblem), _vp, _vp, _vp, ctypes.c_int32, _vp, _vp, _vp],
    "moe_permute_workspace_size": [ctypes.POINTER(MoeProblem), ctypes.POINTER(ctypes.c_size_t)],
    "moe_permute": [ctypes.POINTER(MoeProblem), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                    _vp],
    "moe_grouped_ffn_workspace_size": [ctypes.POINTER(MoeProblem), ctypes.c_int32, ctypes.c_int32,
                                       ctypes.POINTER(ctypes.c_size_t)],
    "moe_grouped_ffn": [ctypes.POINTER(MoeProblem), ctypes.c_int32, ctypes.c_int32, _vp, _vp, _vp,
                        _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp],
    "moe_combine": [ctypes.POINTER(MoeProblem), _vp, _vp, _vp, _vp, _vp, _vp],
    "moe_layer_workspace_size": [ctypes.POINTER(MoeProblem), ctypes.POINTER(ctypes.c_size_t)],
    "moe_layer_plan": [ctypes.POINTER(MoeProblem), ctypes.POINTER(MoePlan)],
    "moe_layer": [ctypes.POINTER(MoeProblem), ctypes.POINTER(MoeLayerArgs), _vp, ctypes.c_size_t, _vp],
    "moe_layer_noalloc_max_bytes": [],
    "moe_layer_noalloc": [ctypes.POINTER(MoeProblem), ctypes.POINTER(MoeLayerArgs), _vp],
    "moe_status_string": [ctypes.c_int],
    "moe_timing_enable": [ctypes.c_int32],
    "moe_timing_read": [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32), ctypes.c_int32],
    "moe_stage_count": [],
    "moe_stage_name": [ctypes.c_int32],
    "moe_debug_fp8_to_bf16": [_vp, _vp, ctypes.c_int32, _vp],
    "moe_debug_f32_to_fp8": [_vp, _vp, ctypes.c_int32, _vp],
    "moe_probe_hbm_read": [_vp, ctypes.c_int64, _vp, _vp],
    "moe_probe_mfma_sink_floats": [],
    "moe_probe_mfma": [ctypes.c_int32, _vp, ctypes.c_int32, _vp, ctypes.POINTER(ctypes.c_double), _vp],
    "moe_quantize_rows": [_vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, _vp, _vp, _vp],
    "moe_quantize_rows_mx": [_vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, _vp, _vp, _vp],
    "moe_quantize_subchannel": [_vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, _vp, _vp, _vp],
}


def lib():
    """The loaded library (loaded once); raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise MoeLibraryMissing(
                f"{LIB_PATH} is not built: run `python -m sparse_mixture_experts_moe_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, argt in _SIG.items():
            f = getattr(L, name)
            f.argtypes = argt
            f.restype = ctypes.c_int
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_layer_noalloc_max_bytes.restype = ctypes.c_size_t
        L.moe_stage_name.restype = ctypes.c_char_p
        _LIB = L
    return _LIB


def exported_symbols():
    return list(_SIG)


def _p(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where)


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def make_problem(T, D, E, k, I, I_shared=0, act="silu", act_shared="silu", act_dtype="bf16",
                 w_dtype="bf16", shared_w_dtype=None, tile_policy="auto",
                 renormalize=True, act_quant=MOE_ACT_QUANT_NONE, combine="auto") -> MoeProblem:
    return MoeProblem(T, D, E, k, I, I_shared, ACTS[act], ACTS[act_shared], int(bool(renormalize)),
                      DTYPES[act_dtype], DTYPES[w_dtype],
                      DTYPES[shared_w_dtype or w_dtype], POLICIES[tile_policy], int(act_quant),
                      COMBINES[combine])


def moe_route(p: MoeProblem, x, w_router, logits, logits_given: bool, topk_idx, topk_w,
              stream=None):
    _check(lib().moe_route(ctypes.byref(p), _p(x), _p(w_router), _p(logits), int(bool(logits_given)),
                           _p(topk_idx), _p(topk_w), _stream(stream)), "moe_route")


def moe_permute_workspace_size(p: MoeProblem) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_permute_workspace_size(ctypes.byref(p), ctypes.byref(n)),
           "moe_permute_workspace_size")
    return n.value


def moe_permute(p: MoeProblem, topk_idx, counts, offsets, row_token, row_of_slot, ws, ws_bytes,
                stream=None, x=None, x_perm=None):
    _check(lib().moe_permute(ctypes.byref(p), _p(topk_idx), _p(counts), _p(offsets), _p(row_token),
                             _p(row_of_slot), _p(x), _p(x_perm), _p(ws), ws_bytes, _stream(stream)),
           "moe_permute")


def moe_grouped_ffn_workspace_size(p: MoeProblem, n_groups: int, rows_upper_bound: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_grouped_ffn_workspace_size(ctypes.byref(p), n_groups, rows_upper_bound,
                                                ctypes.byref(n)), "moe_grouped_ffn_workspace_size")
    return n.value


def moe_grouped_ffn(p: MoeProblem, n_groups: int, rows_upper_bound: int, a, row_token, offsets,
                    w13, s13, w2, s2, h, out, ws, ws_bytes, stream=None):
    _check(lib().moe_grouped_ffn(ctypes.byref(p), n_groups, rows_upper_bound, _p(a), _p(row_token),
                                 _p(offsets), _p(w13), _p(s13), _p(w2), _p(s2), _p(h), _p(out),
                                 _p(ws), ws_bytes, _stream(stream)), "moe_grouped_ffn")


def moe_combine(p: MoeProblem, o_perm, row_of_slot, topk_w, shared_out, y, stream=None):
    _check(lib().moe_combine(ctypes.byref(p), _p(o_perm), _p(row_of_slot), _p(topk_w),
                             _p(shared_out), _p(y), _stream(stream)), "moe_combine")


def moe_layer_workspace_size(p: MoeProblem) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_layer_workspace_size(ctypes.byref(p), ctypes.byref(n)), "moe_layer_workspace_size")
    return n.value


def moe_layer_plan(p: MoeProblem) -> dict:
    """The kernel shape of each product moe_layer runs for p (host planning
    only): router / gate_up / down by name (PLAN_SHAPES), the router's K
    slices, and whether the permutation is one launch."""
    out = MoePlan()
    _check(lib().moe_layer_plan(ctypes.byref(p), ctypes.byref(out)), "moe_layer_plan")
    return {"router": PLAN_SHAPES[out.router], "router_slices": out.router_slices,
            "gate_up": PLAN_SHAPES[out.gate_up], "down": PLAN_SHAPES[out.down],
            "one_launch_permute": bool(out.one_launch_permute)}


def layer_args(**kw) -> MoeLayerArgs:
    a = MoeLayerArgs()
    for name, _ in MoeLayerArgs._fields_:
        setattr(a, name, _p(kw.pop(name, None)))
    if kw:
        raise TypeError(f"unknown moe_layer arguments: {sorted(kw)}")
    return a


def moe_layer(p: MoeProblem, args: MoeLayerArgs, ws, ws_bytes: int, stream=None):
    _check(lib().moe_layer(ctypes.byref(p), ctypes.byref(args), _p(ws), ws_bytes, _stream(stream)),
           "moe_layer")


def moe_layer_noalloc_max_bytes() -> int:
    return lib().moe_layer_noalloc_max_bytes()


def moe_layer_noalloc(p: MoeProblem, args: MoeLayerArgs, stream=None):
    _check(lib().moe_layer_noalloc(ctypes.byref(p), ctypes.byref(args), _stream(stream)), "moe_layer_noalloc")


def moe_timing_enable(on: bool, stages=None):
    """Enable per-stage event timing; `stages` (an iterable of stage indices)
    restricts it to those stages."""
    if on and stages is not None:
        mask = 0
        for st in stages:
            mask |= 1 << int(st)
        val = -(1 << 31) | (mask & 0x7FFFFFFF)
    else:
        val = int(bool(on))
    _check(lib().moe_timing_enable(val), "moe_timing_enable")


def moe_stage_count() -> int:
    return lib().moe_stage_count()


def moe_stage_name(i: int) -> str:
    return lib().moe_stage_name(i).decode()


def moe_timing_read():
    """{stage name: (total ms, launches)} recorded since the last read."""
    n = moe_stage_count()
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int32 * n)()
    _check(lib().moe_timing_read(ms, cnt, n), "moe_timing_read")
    return {moe_stage_name(i): (ms[i], cnt[i]) for i in range(n)}


def moe_quantize_rows(a, rows: int, cols: int, lda: int, q, scale, stream=None):
    _check(lib().moe_quantize_rows(_p(a), rows, cols, lda, _p(q), _p(scale), _stream(stream)),
           "moe_quantize_rows")


def moe_quantize_rows_mx(a, rows: int, cols: int, lda: int, q, scale, stream=None):
    _check(lib().moe_quantize_rows_mx(_p(a), rows, cols, lda, _p(q), _p(scale), _stream(stream)),
           "moe_quantize_rows_mx")


def moe_quantize_subchannel(a, rows: int, cols: int, lda: int, q, scale, stream=None):
    _check(lib().moe_quantize_subchannel(_p(a), rows, cols, lda, _p(q), _p(scale), _stream(stream)),
           "moe_quantize_subchannel")


def moe_probe_hbm_read(buf, nbytes: int, sink, stream=None):
    _check(lib().moe_probe_hbm_read(_p(buf), nbytes, _p(sink), _stream(stream)), "moe_probe_hbm_read")


def moe_probe_mfma_sink_floats() -> int:
    return lib().moe_probe_mfma_sink_floats()


def moe_probe_mfma(dtype: str, operands, iters: int, sink, stream=None) -> float:
    """Launches the MFMA probe; returns the launch's FLOP count."""
    flop = ctypes.c_double(0.0)
    _check(lib().moe_probe_mfma(DTYPES[dtype], _p(operands), iters, _p(sink), ctypes.byref(flop),
                                _stream(stream)), "moe_probe_mfma")
    return flop.value


def moe_debug_fp8_to_bf16(codes, out, n: int, stream=None):
    _check(lib().moe_debug_fp8_to_bf16(_p(codes), _p(out), n, _stream(stream)), "moe_debug_fp8_to_bf16")


def moe_debug_f32_to_fp8(v, out, n: int, stream=None):
    _check(lib().moe_debug_f32_to_fp8(_p(v), _p(out), n, _stream(stream)), "moe_debug_f32_to_fp8")


_OUTS = {"logits_out": ("E", "f32"), "topk_idx_out": ("k", "i32"), "topk_w_out": ("k", "f32"),
         "counts_out": ("E1", "i32"), "offsets_out": ("E2", "i32"),
         "row_token_out": ("Tk", "i32"), "row_of_slot_out": ("Tk", "i32")}


def run_layer(p: MoeProblem, x, w13, w2, w_router=None, s13=None, s2=None, w13_shared=None,
              s13_shared=None, w2_shared=None, s2_shared=None, logits_in=None, want=(),
              ws=None, y=None, stream=None) -> dict:
    """Allocate y, the requested optional outputs and the workspace with torch on
    x's device, call moe_layer once, and return them ({"y": ..., name: ...})."""
    import torch
    dev = x.device
    if y is None:
        y = torch.empty((p.T, p.D), dtype=x.dtype, device=dev)
    outs = {}
    for name in want:
        dim, dt = _OUTS[name]
        shape = {"E": (p.T, p.E), "k": (p.T, p.k), "E1": (p.E,), "E2": (p.E + 1,),
                 "Tk": (p.T * p.k,)}[dim]
        outs[name] = torch.empty(shape, dtype=torch.float32 if dt == "f32" else torch.int32, device=dev)
    need = moe_layer_workspace_size(p)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    args = layer_args(x=x, w_router=w_router, logits_in=logits_in, w13=w13, s13=s13, w2=w2, s2=s2,
                      w13_shared=w13_shared, s13_shared=s13_shared, w2_shared=w2_shared,
                      s2_shared=s2_shared, y=y, **outs)
    moe_layer(p, args, ws, ws.numel(), stream)
    res = {"y": y}
    res.update({k[:-4]: v for k, v in outs.items()})
    return res
