#!/usr/bin/env python3
"""Benchmark of the MXFP4 MoE layer and the MXFP4 quantizer on one MI355X.

A step is one MoE layer forward on the prefill-shaped workload (8192 bf16 tokens, 128 experts, top-8,
hidden 2048, intermediate 768, MXFP4 weights): activation split, routing, pair sort, first grouped
GEMM + SwiGLU, second grouped GEMM + weighted combine, bf16 output.  `value` is algorithmic TFLOP/s
of that layer (2 * T * k * 3 * H * I flops per step).  The same run times the quantizer on the
8192 x 7168 bf16 matrix (GB/s of algorithmic traffic), the decode-shaped layer and the large-expert
layer (4096 tokens, 384 experts, hidden 7168, intermediate 2048, Zipf-skewed routing), and times the
CPU oracle on the same prefill workload as a reported baseline.  Inputs are synthetic and seeded; weights are
quantized from random bf16 masters.  Prints one JSON line.
"""

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import mixed_precision_moe_amd as mx  # noqa: E402
from mixed_precision_moe_amd import synth  # noqa: E402
from mixed_precision_moe_amd._lib import MoeDims, check, lib  # noqa: E402
from tests.gpu_common import bf16_dev, gpu_standard_weights  # noqa: E402

PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
PEAK_FP4_TFLOPS = 10100.0  # MI355X dense MXFP4 / MXFP6 MFMA
# the forward's stages as the library's events bracket them, and the kernels each stage launches
STAGES = ["act_split", "route", "pair_sort", "gemm1_swiglu", "gemm2_weighted", "combine"]
STAGE_KERNELS = ["xprep_kernel", "route_kernel", "place_kernel", "grouped_gemm_kernel<G1=true>",
                 "grouped_gemm_kernel<G1=false>", "combine_kernel"]
DTYPE = "mxfp4 (e2m1 + e8m0) weights x two-term e2m3 (fp6) activations on block-scaled MFMA, fp32 accumulate"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_prefill_gemm1_and_quantize.txt")


def measured_traffic(which):
    """HBM bytes per launch of `which` ("gemm" = the first GEMM on the prefill workload, or "quantize")
    from the committed counter summary (FETCH_SIZE + WRITE_SIZE, each scaled by the same counter on a
    copy of known size), or None when the summary is missing or the kernel's source file has changed
    since the counters were taken."""
    import hashlib
    key = {"gemm": ("traffic_bytes_per_launch", "gemm_source_sha256", "gemm.hip"),
           "quantize": ("quantize_traffic_bytes_per_launch", "quantize_source_sha256", "quantize.hip")}[which]
    try:
        fields = dict(l.split(None, 1) for l in open(TRAFFIC_FILE).read().splitlines() if l.strip() and not l.startswith("#"))
        src = open(os.path.join(ROOT, "mixed_precision_moe_amd", "csrc", key[2]), "rb").read()
        if hashlib.sha256(src).hexdigest() != fields[key[1]].strip():
            return None
        return float(fields[key[0]])
    except (OSError, KeyError, ValueError):
        return None


def moe_flops(cfg):
    return 2.0 * cfg.T * cfg.k * 3 * cfg.H * cfg.I


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class MoeBench:
    def __init__(self, cfg, rotations, weight_copies=None, act=0):
        self.cfg = cfg
        self.act = act
        w = gpu_standard_weights(cfg)
        self.packed = [mx.repack_weights(*w)]
        # extra weight copies so consecutive steps cannot hit in the 256 MB cache (not needed once the
        # weights alone are many times that size)
        for _ in range(1, rotations if weight_copies is None else weight_copies):
            self.packed.append(self.packed[0].clone())
        del w
        x_bits, logits = synth.moe_activations(cfg)
        self.x = [bf16_dev(x_bits) for _ in range(rotations)]
        self.logits = [torch.from_numpy(logits).cuda() for _ in range(rotations)]
        self.y = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda")
        self.d = MoeDims(cfg.E, cfg.H, cfg.I, 1 if cfg.bias else 0)
        import ctypes
        self.ctypes = ctypes
        nws = lib().moe_mxfp4_workspace_bytes(ctypes.byref(self.d), cfg.T, cfg.k)
        self.ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
        self.stream = torch.cuda.current_stream()
        self.i = 0

    def step(self, events=None):
        c = self.ctypes
        r = self.i % len(self.x)
        self.i += 1
        args = [c.byref(self.d), self.act, c.c_void_p(self.packed[r % len(self.packed)].data_ptr()),
                c.c_void_p(self.x[r].data_ptr()),
                self.cfg.T, self.cfg.H, c.c_void_p(self.logits[r].data_ptr()), self.cfg.k,
                1 if self.cfg.renormalize else 0, c.c_void_p(self.y.data_ptr()), None, None,
                c.c_void_p(self.ws.data_ptr()), self.ws.numel(), c.c_void_p(self.stream.cuda_stream)]
        if events is None:
            check("moe_mxfp4_forward_act", lib().moe_mxfp4_forward_act(*args))
        else:
            arr = (c.c_void_p * len(events))(*events)
            check("moe_mxfp4_forward_profiled", lib().moe_mxfp4_forward_profiled(*args, arr, len(events)))


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence (hip_runtime_api.h)


class HipEvents:
    """Raw HIP events (recorded by the library itself on its stream).  They only time: created with
    hipEventDisableSystemFence, a record does not write back and invalidate the caches, which would
    otherwise add several microseconds per stage boundary to the measured step."""

    def __init__(self, n):
        import ctypes
        self.c = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            assert self.hip.hipEventCreateWithFlags(ctypes.byref(h), ctypes.c_uint(HIP_EVENT_DISABLE_SYSTEM_FENCE)) == 0
            self.ev.append(h)

    def elapsed_ms(self, a, b):
        f = self.c.c_float()
        assert self.hip.hipEventElapsedTime(self.c.byref(f), self.ev[a], self.ev[b]) == 0
        return f.value

    def __del__(self):
        for h in getattr(self, "ev", []):
            self.hip.hipEventDestroy(h)


def time_moe(b, steps, warmup):
    for _ in range(warmup):
        b.step()
    ns = len(STAGES) + 1
    evs = HipEvents(steps * ns)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        b.step(evs.ev[s * ns:(s + 1) * ns])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    per_stage = np.zeros(len(STAGES))
    for s in range(steps):
        for j in range(len(STAGES)):
            per_stage[j] += evs.elapsed_ms(s * ns + j, s * ns + j + 1)
    per_stage /= steps
    return (t1 - t0) * 1e3 / steps, per_stage


def bench_quantize(steps, warmup, rotations=4):
    M, K = synth.QUANT_CONFIG["M"], synth.QUANT_CONFIG["K"]
    bits = synth.quant_matrix(M, K, cid=synth.QUANT_CONFIG["cid"])
    xs = [bf16_dev(bits) for _ in range(rotations)]
    qs = [torch.empty((M, K // 2), dtype=torch.uint8, device="cuda") for _ in range(rotations)]
    sfs = [torch.empty((M, K // 32), dtype=torch.uint8, device="cuda") for _ in range(rotations)]
    sts = [torch.empty(mx.tiled_scale_shape(M, K), dtype=torch.uint8, device="cuda") for _ in range(rotations)]
    L = lib()
    import ctypes
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = [(ctypes.c_void_p(xs[r].data_ptr()), ctypes.c_void_p(qs[r].data_ptr()), ctypes.c_void_p(sfs[r].data_ptr()),
             ctypes.c_void_p(sts[r].data_ptr())) for r in range(rotations)]

    def one(i):
        a = args[i % rotations]
        check("mxfp4_quantize", L.mxfp4_quantize(a[0], M, K, K, a[1], a[2], a[3], st))
    for i in range(warmup):
        one(i)
    n = max(steps, 20)
    # The launches are queued behind a GPU-side sleep, so the host has enqueued all of them before the
    # first runs: the interval between the two events is n launches back to back on the stream they
    # run on, without gaps from host-side launch overhead.
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    torch.cuda._sleep(20_000_000)
    ev[0].record()
    for i in range(n):
        one(i)
    ev[1].record()
    torch.cuda.synchronize()
    ms = float(ev[0].elapsed_time(ev[1])) / n
    nbytes = M * K * 2 + M * K // 2 + 2 * (M * K // 32)  # bf16 in, nibbles, flat + tiled scales (no padding here)
    return {"workload": f"quantize bf16 {M}x{K} -> E2M1 nibbles + E8M0 flat and tiled scales", "ms": ms,
            "bytes": nbytes, "GB_s": nbytes / (ms * 1e-3) / 1e9, "launches": n}


def cpu_baselines(cfg, x_bits, logits):
    """The oracle, untuned, on bounded samples of the two workloads."""
    from oracle import moe as M
    from oracle import quant as Q
    from tests.gpu_common import LazyExperts
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = None
    cores = len(os.sched_getaffinity(0))
    # MoE: the whole prefill workload (every token); the oracle dequantizes every expert the routing
    # uses in fp64, which dominates its time (about 5-25 s on 8-16 host cores)
    ntok = cfg.T
    rows = np.arange(ntok)
    w13, w2 = LazyExperts(cfg, "w13"), LazyExperts(cfg, "w2")
    from oracle.route import route_ref
    ids, _ = route_ref(logits, cfg.k)
    from concurrent.futures import ThreadPoolExecutor
    from tests.gpu_common import workers
    with ThreadPoolExecutor(workers()) as ex:  # quantizing the masters is input preparation, not timed
        list(ex.map(lambda e: (w13.get(e), w2.get(e)), np.unique(ids[rows])))
    t0 = time.perf_counter()
    M.moe_ref(x_bits, logits, cfg.k, w13.q, w13.s, w2.q, w2.s, None, None, tokens=rows)
    dt = time.perf_counter() - t0
    flops = 2.0 * ntok * cfg.k * 3 * cfg.H * cfg.I
    moe = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "blas_threads": blas_threads,
           "kind": "oracle", "seconds": dt,
           "sample": f"all {ntok} prefill tokens ({len(np.unique(ids[rows]))} experts used, dequantized in fp64); "
                     "weights pre-quantized outside the timed region"}
    # quantizer: the whole 8192 x 7168 matrix
    Mq, K = synth.QUANT_CONFIG["M"], synth.QUANT_CONFIG["K"]
    sub = synth.quant_matrix(Mq, K, cid=synth.QUANT_CONFIG["cid"])
    t0 = time.perf_counter()
    q, s = Q.quantize_ref(sub)
    Q.tile_scales(s)
    dt = time.perf_counter() - t0
    nbytes = Mq * K * 2 + Mq * K // 2 + 2 * Mq * K // 32
    quant = {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle", "seconds": dt,
             "sample": f"all {Mq} rows of the quantize matrix"}
    return moe, quant


def run_quantize(args):
    log("[bench] timing quantize")
    qr = bench_quantize(args.steps, args.warmup)
    qr["roofline"] = {"bound": "hbm", "kernel": "quantize_kernel", "achieved": qr["GB_s"], "peak": PEAK_HBM_GBS,
                      "unit": "GB/s", "frac": qr["GB_s"] / PEAK_HBM_GBS, "traffic": measured_traffic("quantize")}
    return qr


def touched_experts(b):
    """Number of distinct experts the workload's routing selects, from the library's own routing."""
    ids = mx.route(b.logits[0], b.cfg.k, b.cfg.renormalize)[0]
    return int(torch.unique(ids).numel())


def expert_bytes(cfg):
    """Packed MXFP4 bytes of one expert: w13 and w2 nibbles and E8M0 scales, plus bf16 biases."""
    n = 2 * cfg.I * cfg.H // 2 + 2 * cfg.I * cfg.H // 32 + cfg.H * cfg.I // 2 + cfg.H * cfg.I // 32
    return n + (2 * (2 * cfg.I + cfg.H) if cfg.bias else 0)


def run_decode(args):
    dcfg = synth.MOE_CONFIGS["decode"]
    log("[bench] timing decode MoE")
    db = MoeBench(dcfg, rotations=2)
    dms, dstages = time_moe(db, max(args.steps, 50), args.warmup)
    touched = touched_experts(db)
    nbytes = touched * expert_bytes(dcfg) + dcfg.T * dcfg.H * 4 + dcfg.T * dcfg.E * 4
    return {"workload": "decode-shaped MXFP4 MoE layer (T=64, E=128, top-8, H=2048, I=768, biases)",
            "ms": dms, "stages_ms": {n: float(v) for n, v in zip(STAGES, dstages)},
            "touched_experts": touched, "algorithmic_bytes": nbytes,
            "GB_s": nbytes / (dms * 1e-3) / 1e9, "frac_of_hbm": nbytes / (dms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "TFLOP_s": moe_flops(dcfg) / (dms * 1e-3) / 1e12}


def run_large(args):
    lcfg = synth.MOE_CONFIGS["large"]
    log(f"[bench] building large-expert workload T={lcfg.T} E={lcfg.E} k={lcfg.k} H={lcfg.H} I={lcfg.I}")
    lb = MoeBench(lcfg, rotations=2, weight_copies=1)  # 9 GB of weights: nothing survives in the cache
    log("[bench] timing large-expert MoE")
    lms, lstages = time_moe(lb, args.steps, args.warmup)
    touched = touched_experts(lb)
    P = lcfg.T * lcfg.k
    # touched weights, x, logits, y, and the SwiGLU activation written and read once in bf16
    nbytes = touched * expert_bytes(lcfg) + lcfg.T * lcfg.H * 4 + lcfg.T * lcfg.E * 4 + P * lcfg.I * 4
    tflops = moe_flops(lcfg) / (lms * 1e-3) / 1e12
    return {"workload": "large-expert MXFP4 MoE layer (T=4096, E=384, top-8, H=7168, I=2048, Zipf(1.2) routing)",
            "ms": lms, "stages_ms": {n: float(v) for n, v in zip(STAGES, lstages)},
            "touched_experts": touched, "algorithmic_bytes": nbytes,
            "GB_s": nbytes / (lms * 1e-3) / 1e9, "frac_of_hbm": nbytes / (lms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "TFLOP_s": tflops, "frac_of_fp4_peak": tflops / PEAK_FP4_TFLOPS}


def only_secondary(args):
    out = {"metric": "MXFP4 MoE layer TFLOP/s + quantize GB/s, % of MI355X roofline, 1 GPU", "only": args.only}
    if args.only == "decode":
        out["decode"] = run_decode(args)
    elif args.only == "large":
        out["large"] = run_large(args)
    else:
        out["quantize"] = run_quantize(args)
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-quantize", action="store_true")
    ap.add_argument("--no-large", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode", "quantize", "large"], default=None,
                    help="time one workload only (for profiler runs); the JSON line then holds that workload")
    args = ap.parse_args()
    if args.only == "prefill":
        args.no_decode = args.no_quantize = args.no_large = args.no_cpu_baseline = True
    elif args.only == "decode":
        args.no_quantize = args.no_cpu_baseline = True
    elif args.only == "quantize":
        args.no_decode = args.no_cpu_baseline = True
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this library has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "needs a GPU"
    torch.cuda.set_device(0)

    cfg = synth.MOE_CONFIGS["prefill"]
    if args.only in ("decode", "quantize", "large"):
        return only_secondary(args)
    log(f"[bench] building prefill workload T={cfg.T} E={cfg.E} k={cfg.k} H={cfg.H} I={cfg.I}")
    b = MoeBench(cfg, rotations=2)
    log("[bench] timing prefill MoE")
    ms, stages = time_moe(b, args.steps, args.warmup)
    flops = moe_flops(cfg)
    value = flops / (ms * 1e-3) / 1e12
    P = cfg.T * cfg.k
    g1_flops = 2.0 * P * cfg.H * 2 * cfg.I
    g2_flops = 2.0 * P * cfg.I * cfg.H
    g1_ms, g2_ms = stages[3], stages[4]
    # the dominant kernel: algorithmic flops of the first GEMM per launch over its measured launch time
    # (HIP events the library records on its own stream around the launch).  The MFMA issues every
    # product once per activation term, so the matrix cores execute twice the algorithmic flops.
    g1_tf = g1_flops / (g1_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": "grouped_gemm_kernel<G1=true> (first grouped GEMM + SwiGLU)",
                "achieved": g1_tf, "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s", "frac": g1_tf / PEAK_FP4_TFLOPS,
                "traffic": measured_traffic("gemm"), "flops_per_launch": g1_flops, "avg_launch_ms": g1_ms,
                "mfma_issued_frac": 2 * g1_tf / PEAK_FP4_TFLOPS}
    out = {
        "metric": "MXFP4 MoE layer TFLOP/s + quantize GB/s, % of MI355X roofline, 1 GPU",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": DTYPE, "data": "synthetic",
        "config": {"workload": "prefill-shaped MXFP4 MoE layer, bf16 tokens", "T": cfg.T, "E": cfg.E, "top_k": cfg.k,
                   "H": cfg.H, "I": cfg.I, "bias": cfg.bias, "parallelism": "single GPU"},
        "roofline": roofline,
        "stages_ms": {n: float(v) for n, v in zip(STAGES, stages)},
        "layer_frac_of_fp4_peak": value / PEAK_FP4_TFLOPS,
        "stage_kernels": dict(zip(STAGES, STAGE_KERNELS)),
        "gemm2": {"achieved_TFLOP_s": g2_flops / (g2_ms * 1e-3) / 1e12, "avg_launch_ms": g2_ms},
    }
    x_bits_host, logits_host = synth.moe_activations(cfg)
    del b
    torch.cuda.empty_cache()

    if not args.no_quantize:
        out["quantize"] = run_quantize(args)
        torch.cuda.empty_cache()

    if not args.no_decode:
        out["decode"] = run_decode(args)
        torch.cuda.empty_cache()

    if not args.no_large:
        out["large"] = run_large(args)
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        moe_cpu, q_cpu = cpu_baselines(cfg, x_bits_host, logits_host)
        out["cpu_baseline"] = moe_cpu
        if "quantize" in out:
            out["quantize"]["cpu_baseline"] = q_cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
