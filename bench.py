"""Benchmark of the routed MoE FFN layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one call of moe_layer (router -> top-k softmax -> permutation ->
grouped gate/up+activation -> grouped down projection -> combine with the
shared branch) over one batch of synthetic tokens whose inputs are already in
HBM.  Prints one JSON line: whole-job tokens/s, the dominant kernel's roofline
fraction (algorithmic bytes or FLOP per launch over its average event-timed
duration) and the CPU oracle timed on a bounded sample of the same workload.

A short diagnostic pass first times every stage between HIP event pairs (the
per-stage breakdown, and which stage dominates); the timed region then brackets
only the dominant stage with events, since each event pair costs a few
microseconds of stream time that would otherwise inflate the layer time.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# The largest configuration that fits one GPU and the one the prefill MFMA
# target is quoted on: the Ling-2.6-1T-style layer at 16384 tokens, fp8
# per-channel expert weights with bf16 activations (W8A16).
DEFAULT_WORKLOAD = "ling_prefill"
METRIC = "MoE-layer tokens/s; grouped-GEMM MFMA % of peak (prefill), HBM % (decode)"


def sources_hash(files) -> str:
    """sha256 over the given repository files, in order: a traffic record is
    only used while the sources of the kernel it measured are unchanged."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--policy", default="auto", choices=["auto", "stream", "lds"])
    ap.add_argument("--combine", default="auto", choices=["auto", "separate", "fused"],
                    help="where the layer combines the expert rows (default: the library's choice)")
    ap.add_argument("--act-quant", nargs="?", const="row", default=None, choices=["row", "sub512"],
                    help="dynamic fp8 activations in the expert GEMMs (fp8-weight workloads): one scale "
                         "per token row (row, the default), or per 512-element sub-channel (sub512)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0)
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="only run 10 plain device copies of MIB MiB (counter calibration)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured HBM / MFMA ceilings")
    return ap.parse_args()


def copy_calib(mib: int):
    """Ten device-to-device copies of a known size, so HBM counters read under a
    profiler can be scaled to bytes (FETCH_SIZE / WRITE_SIZE per dispatch vs
    the known size)."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calib_bytes": n, "copies": 10}), flush=True)


def cpu_identity():
    """(CPU model, number of cores this process may run on)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def measured_peaks(B, stream):
    """The GPU's own ceilings, measured in this job with the library's probes:
    a streaming read of 4 GiB, and register-only bf16 and fp8 MFMA loops on
    random operands (each launch about 20 ms; median of 5 after 2 warm-ups)."""
    import torch

    def timed(fn, reps=5, warm=2):
        for _ in range(warm):
            fn()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return sorted(ts)[len(ts) // 2]

    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    t = timed(lambda: B.moe_probe_hbm_read(buf, nbytes, sink, stream))
    hbm = nbytes / t / 1e9
    del buf
    g = torch.Generator().manual_seed(0)
    ops = torch.randn(65536, generator=g)
    fs = torch.empty(B.moe_probe_mfma_sink_floats(), dtype=torch.float32, device="cuda")
    out = {"hbm_read_GBps": hbm}
    for dt, o, iters in (("bf16", ops[:32768].to(torch.bfloat16), 37000),
                         ("fp8", ops.to(torch.float8_e4m3fn), 18600)):
        od = o.view(torch.uint8).cuda()
        flop = [0.0]

        def run():
            flop[0] = B.moe_probe_mfma(dt, od, iters, fs, stream)
        t = timed(run)
        out[f"mfma_{dt}_TFLOPs"] = flop[0] / t / 1e12
    return out


MIN_CPU_S, MAX_CPU_S = 10.0, 30.0   # CPU baseline: seconds of oracle work


def cpu_baseline(wl, n_tokens: int, act_quant: int = 0):
    """Time the oracle (as it stands) on the first n_tokens tokens of the batch:
    routing of those tokens, every expert they touch, the shared branch and
    the combine, with expert weights decoded from their stored format inside
    the timed region.  Host copies of the raw inputs are made beforehand."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle.actquant import layer_w8a8
    from oracle.formats import decode
    from oracle.moe import layer
    from oracle.mx import decode_weight, layer_w4a8
    from workloads import host_expert, host_shared, to_bits

    c = wl.cfg
    xb = to_bits(wl.x[:n_tokens])
    wrb = to_bits(wl.wr)
    # routing of the sample decides which experts the oracle needs
    x64 = decode(xb, c.act_dtype)
    wr64 = decode(wrb, c.act_dtype)
    from oracle.moe import router_logits, topk_softmax
    idx, _ = topk_softmax(router_logits(x64, wr64), c.k)
    used = sorted(set(int(e) for e in idx.reshape(-1)))
    raw = {e: host_expert(wl, e) for e in used}
    sh = host_shared(wl)

    def expert(e):
        w13, s13, w2, s2 = raw[e]
        return (*decode_weight(w13, s13, c.w_dtype), *decode_weight(w2, s2, c.w_dtype))

    def one_pass():
        x = decode(xb, c.act_dtype)
        wr = decode(wrb, c.act_dtype)
        shared = None
        if sh is not None:
            shared = (*decode_weight(sh[0], sh[1], c.shared_w_dtype),
                      *decode_weight(sh[2], sh[3], c.shared_w_dtype))
        if act_quant == 3:
            layer_w8a8(x, wr, c.k, expert, shared, c.act, c.act_shared, width=512)
        else:
            fn = {0: layer, 1: layer_w8a8, 2: layer_w4a8}[act_quant]
            fn(x, wr, c.k, expert, shared, c.act, c.act_shared)

    # whole passes over the sample until at least MIN_CPU_S seconds of work
    t0 = time.perf_counter()
    passes = 0
    while True:
        one_pass()
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= MIN_CPU_S or dt / passes * (passes + 1) > MAX_CPU_S:
            break
    threads = 1
    for info in threadpool_info():
        if info.get("user_api") == "blas":
            threads = max(threads, int(info.get("num_threads", 1)))
    model, affinity = cpu_identity()
    return {"value": passes * n_tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": model, "cpus_available": affinity,
            "sample": (f"float64 NumPy oracle{['', ' (W8A8)', ' (W4A8)', ' (W8A8, 512-element sub-channels)'][act_quant]}, whole layer on the "
                       f"first {n_tokens} of {c.T} tokens "
                       f"({len(used)} experts decoded from {c.w_dtype} in each pass), "
                       f"{passes} pass{'es' if passes > 1 else ''}, {dt:.1f} s")}


def main():
    args = parse()
    if args.copy_calib:
        copy_calib(args.copy_calib)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the layer runs on one GPU here; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    from sparse_mixture_experts_moe_amd import binding as B
    from sparse_mixture_experts_moe_amd import costmodel as cm
    from workloads import CONFIGS, generate

    B.lib()  # fails loudly if the HIP library is not built
    cfg = CONFIGS[args.workload]
    torch.cuda.set_device(0)
    wl = generate(cfg, seed=0, weight_device="cuda")
    wl.x, wl.wr = wl.x.cuda(), wl.wr.cuda()
    # MXFP4 weights always run with MXFP8 activations (W4A8)
    aq = (B.MOE_ACT_QUANT_MXFP8 if cfg.w_dtype == "mxfp4"
          else B.MOE_ACT_QUANT_FP8_ROW if args.act_quant == "row"
          else B.MOE_ACT_QUANT_FP8_SUB if args.act_quant == "sub512" else B.MOE_ACT_QUANT_NONE)
    p = B.make_problem(cfg.T, cfg.D, cfg.E, cfg.k, cfg.I, cfg.I_shared, cfg.act, cfg.act_shared,
                       cfg.act_dtype, cfg.w_dtype, cfg.shared_w_dtype, args.policy, act_quant=aq,
                       combine=args.combine)
    ws_bytes = B.moe_layer_workspace_size(p)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    y = torch.empty((cfg.T, cfg.D), dtype=wl.x.dtype, device="cuda")
    counts = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    kw = dict(x=wl.x, w_router=wl.wr, w13=wl.w13, s13=wl.s13, w2=wl.w2, s2=wl.s2,
              w13_shared=wl.w13s, s13_shared=wl.s13s, w2_shared=wl.w2s, s2_shared=wl.s2s, y=y)
    step_args = B.layer_args(**kw)
    probe_args = B.layer_args(counts_out=counts, **kw)
    stream = torch.cuda.current_stream()

    B.moe_layer(p, probe_args, ws, ws_bytes, stream)
    torch.cuda.synchronize()
    touched = int((counts.cpu().numpy() > 0).sum())

    for _ in range(args.warmup):
        B.moe_layer(p, step_args, ws, ws_bytes, stream)
    torch.cuda.synchronize()

    # per-stage breakdown (diagnostic pass, every stage between an event pair);
    # it also names the dominant kernel
    diag_steps = min(args.steps, 10)
    B.moe_timing_read()
    B.moe_timing_enable(True)
    for _ in range(diag_steps):
        B.moe_layer(p, step_args, ws, ws_bytes, stream)
    torch.cuda.synchronize()
    B.moe_timing_enable(False)
    diag = B.moe_timing_read()
    stage_names = [B.moe_stage_name(i) for i in range(B.moe_stage_count())]
    name = max(diag.items(), key=lambda kv: kv[1][0])[0]

    # timed region: K steps; HIP events on the layer's stream bracket only the
    # dominant stage, so the other stages run without events between them
    B.moe_timing_enable(True, stages=[stage_names.index(name)])
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for _ in range(args.steps):
        B.moe_layer(p, step_args, ws, ws_bytes, stream)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    B.moe_timing_enable(False)
    stages = B.moe_timing_read()
    total_ms = t0.elapsed_time(t1)
    ms_per_step = total_ms / args.steps
    tokens_per_s = cfg.T * args.steps / (total_ms / 1e3)

    # dominant kernel and its roofline
    st_ms, st_n = stages[name]
    avg_ms = st_ms / max(st_n, 1)
    launches_per_step = st_n / args.steps
    per_launch = {
        "ffn1_gate_up_act": (cm.gemm1_bytes(cfg, touched), cm.gemm1_flops(cfg)),
        "ffn2_down": (cm.gemm2_bytes(cfg, touched), cm.gemm2_flops(cfg)),
    }
    bytes_, flops = per_launch.get(name, (0.0, 0.0))
    bytes_ /= launches_per_step
    flops /= launches_per_step
    ai = flops / bytes_ if bytes_ else 0.0
    # the matrix cores' dtype: fp8 x fp8 with quantised activations; e4m3 x
    # e2m1 (W4A8) issues at the fp8 rate, so its peak is fp8's
    wdt = "fp8" if aq else ("bf16" if cfg.act_dtype == "bf16" else "f32")
    ridge = cm.PEAK_TFLOPS[wdt] * 1e12 / (cm.PEAK_HBM_GBS * 1e9)
    traffic = None
    tpath = os.path.join(ROOT, "profiles",
                         f"traffic_{name}_{cfg.name}{ {1: '_w8a8', 3: '_w8a8sub'}.get(aq, '') }.json")
    if os.path.exists(tpath):
        tj = json.load(open(tpath))
        if tj.get("sources") and tj.get("sources_sha256") == sources_hash(tj["sources"]):
            traffic = tj.get("bytes_per_launch")
    if ai < ridge:
        roof = {"bound": "hbm", "achieved": bytes_ / (avg_ms * 1e-3) / 1e9, "peak": cm.PEAK_HBM_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": flops / (avg_ms * 1e-3) / 1e12,
                "peak": cm.PEAK_TFLOPS[wdt], "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = traffic
    peaks = None if args.no_peaks else measured_peaks(B, stream)
    if peaks:
        m = peaks["hbm_read_GBps"] if roof["bound"] == "hbm" else peaks[f"mfma_{wdt}_TFLOPs"]
        roof["measured_peak"] = m
        roof["frac_of_measured"] = roof["achieved"] / m
    roof.update({"kernel": name, "avg_launch_ms": avg_ms, "algorithmic_bytes": bytes_,
                 "algorithmic_flops": flops})

    gemm_ms = sum(diag[s][0] for s in ("ffn1_gate_up_act", "ffn2_down")) / diag_steps
    out = {
        "metric": METRIC, "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8*fp4" if aq == B.MOE_ACT_QUANT_MXFP8 else wdt, "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "D": cfg.D, "E": cfg.E, "k": cfg.k,
                   "I": cfg.I, "I_shared": cfg.I_shared, "act": cfg.act,
                   "w_dtype": cfg.w_dtype, "touched_experts": touched, "policy": args.policy,
                   "act_quant": ["none", "fp8_per_token", "mxfp8", "fp8_per_512_subchannel"][aq]},
        "roofline": roof,
        "grouped_gemm": {
            "ms_per_step": gemm_ms,
            "mfma_frac_bf16": cm.gemm_flops(cfg) / (gemm_ms * 1e-3) / (cm.PEAK_TFLOPS["bf16"] * 1e12),
            "mfma_frac_fp8": cm.gemm_flops(cfg) / (gemm_ms * 1e-3) / (cm.PEAK_TFLOPS["fp8"] * 1e12),
            "hbm_frac_layer_bytes": cm.layer_bytes(cfg, touched) / (ms_per_step * 1e-3)
            / (cm.PEAK_HBM_GBS * 1e9)},
        "stages_ms_per_step": {k: v[0] / diag_steps for k, v in diag.items()},
        "measured_peaks": peaks,
        "wall_s": wall,
    }
    if not args.no_cpu_baseline:
        # a sample of about 10-30 s of oracle work on the host
        n = args.cpu_sample_tokens or {"qwen_decode": 64, "ling_decode": 16, "ling_prefill": 4,
                                       "ling_prefill_mxfp4": 4}.get(cfg.name, 16)
        out["cpu_baseline"] = cpu_baseline(wl, min(n, cfg.T), aq)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
