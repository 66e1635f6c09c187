#!/usr/bin/env python3
"""Benchmark of the MXFP4 MoE layer and the MXFP4 quantizer on one MI355X.

A step is one MoE layer forward on the prefill-shaped workload (8192 bf16 tokens, 128 experts, top-8,
hidden 2048, intermediate 768, MXFP4 weights): activation split and routing, pair sort, first grouped
GEMM + SwiGLU, second grouped GEMM + weighted combine, bf16 output.  `value` is algorithmic TFLOP/s
of that layer (2 * T * k * 3 * H * I flops per step).

The same run also times, each in an object of its own on the JSON line:
  tiny      the 16-token layer (4 experts, top-2, hidden 256, intermediate 128, biases): latency
  decode    the 64-token layer (128 experts, hidden 2048, intermediate 768, biases): HBM fraction
  large     4096 tokens, 384 experts, hidden 7168, intermediate 2048, Zipf(1.2) routing
  quantize  MXFP4 quantizer on the 8192 x 7168 bf16 matrix: GB/s of algorithmic traffic
  variants  the prefill layer with MXFP8 and with MXFP4 activations
  nvfp4     the NVFP4 quantizer (E4M3 block scales, global scale) on the same 8192 x 7168 matrix
  linear    the dense MXFP4-weight linear layer on 8192 x 7168 x 7168
and, in its CPU leg, times the oracle on each MoE workload (all tokens; the large-expert layer on a
stated sample) and on the quantize matrix, and compares the library's outputs with the oracle's:
max |err| / rms and the count of elements outside |err| <= 2e-2 * rms + 1e-3 per MoE workload,
mismatching bytes and the saturation fraction for the quantizer.  Per-expert load statistics come
from the library's own routing.  Inputs are synthetic and seeded; weights are quantized from random
bf16 masters.  Prints one JSON line.
"""

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import mixed_precision_moe_amd as mx  # noqa: E402
from mixed_precision_moe_amd import synth  # noqa: E402
from mixed_precision_moe_amd._lib import MoeDims, check, lib  # noqa: E402
from tests.gpu_common import ATOL, RTOL_RMS, bf16_dev, bf16_host_f64, gpu_standard_weights, workers  # noqa: E402

METRIC = "MXFP4 MoE layer TFLOP/s + quantize GB/s, % of MI355X roofline, 1 GPU"
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
PEAK_FP4_TFLOPS = 10100.0  # MI355X dense MXFP4 / MXFP6 MFMA
ACT_TERMS = 3              # bf16 activations enter the MFMA as three block-scaled terms
# the forward's stages as the library's events bracket them, and the kernels each stage launches
STAGES = ["split_and_route", "pair_sort", "gemm1_swiglu", "gemm2_weighted", "combine"]
STAGE_KERNELS = ["front_kernel", "place_kernel", "grouped_gemm_kernel<G1=true>", "grouped_gemm_kernel<G1=false>",
                 "combine_kernel"]
DTYPE = ("mxfp4 (e2m1 + e8m0) weights x bf16 activations split into three block-scaled terms "
         "(e2m3, e2m3, e2m1) on scaled MFMA, fp32 accumulate, bf16 out")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_per_kernel.txt")
CSRC = os.path.join(ROOT, "mixed_precision_moe_amd", "csrc")
# the sources each measured kernel is compiled from: a counter figure stands only while they are unchanged
KERNEL_SOURCES = {"gemm": ["gemm_kernel.h", "gemm.hip", "common.h", "layout.h"],
                  "quantize": ["quantize.hip", "common.h", "layout.h"]}
TINY_ITERS = 200
DECODE_ITERS = 100
LARGE_SAMPLE_TOKENS = 4


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def sources_sha256(which):
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[which]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(which):
    """HBM bytes per launch of `which` ("gemm" = the first GEMM on the prefill workload, or "quantize")
    from the committed counter summary (FETCH_SIZE + WRITE_SIZE, each scaled by the same counter on a
    copy of known size), or None when the summary is missing or the kernel's sources have changed
    since the counters were taken."""
    key = {"gemm": ("traffic_bytes_per_launch", "gemm_sources_sha256"),
           "quantize": ("quantize_traffic_bytes_per_launch", "quantize_sources_sha256")}[which]
    try:
        with open(TRAFFIC_FILE) as f:
            fields = dict(l.split(None, 1) for l in f.read().splitlines() if l.strip() and not l.startswith("#"))
        if sources_sha256(which) != fields[key[1]].strip():
            return None
        return float(fields[key[0]])
    except (OSError, KeyError, ValueError):
        return None


def moe_flops(cfg):
    return 2.0 * cfg.T * cfg.k * 3 * cfg.H * cfg.I


def host_cpu():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = None
    return {"model": model, "cores": len(os.sched_getaffinity(0)), "blas_threads": blas}


class MoeBench:
    """One MoE workload on the GPU: packed weights (optionally several copies, so consecutive steps
    stream them from HBM rather than the 256 MB cache), rotating input sets and a workspace."""

    def __init__(self, cfg, rotations, weight_copies=None, act=mx.ACT_BF16):
        self.cfg = cfg
        self.act = act
        w = gpu_standard_weights(cfg)
        self.packed = [mx.repack_weights(*w)]
        for _ in range(1, rotations if weight_copies is None else weight_copies):
            self.packed.append(self.packed[0].clone())
        del w
        self.x_bits, self.logits_host = synth.moe_activations(cfg)
        self.x = [bf16_dev(self.x_bits) for _ in range(rotations)]
        self.logits = [torch.from_numpy(self.logits_host).cuda() for _ in range(rotations)]
        self.y = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda")
        self.d = MoeDims(cfg.E, cfg.H, cfg.I, 1 if cfg.bias else 0)
        nws = lib().moe_mxfp4_workspace_bytes(ctypes.byref(self.d), cfg.T, cfg.k)
        self.ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
        self.stream = torch.cuda.current_stream()
        self.i = 0

    def step(self, events=None):
        c = ctypes
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

    def outputs(self):
        """y of the last step as float64 on the host (every rotation holds the same inputs), with the
        host copies of the inputs."""
        torch.cuda.synchronize()
        return {"y": bf16_host_f64(self.y), "x_bits": self.x_bits, "logits": self.logits_host}

    def expert_load(self):
        """Pairs per expert under the library's own routing of the workload."""
        ids = mx.route(self.logits[0], self.cfg.k, self.cfg.renormalize)[0]
        cnt = np.bincount(ids.cpu().numpy().ravel(), minlength=self.cfg.E)
        return {"pairs": int(cnt.sum()), "experts": self.cfg.E, "experts_used": int(np.count_nonzero(cnt)),
                "min": int(cnt.min()), "max": int(cnt.max()), "mean": float(cnt.mean()),
                "median": float(np.median(cnt)), "std": float(cnt.std()),
                "max_over_mean": float(cnt.max() / cnt.mean()),
                "top5": [int(v) for v in np.sort(cnt)[::-1][:5]],
                "experts_below_32_pairs": int(np.count_nonzero(cnt < 32))}


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence (hip_runtime_api.h)


class HipEvents:
    """Raw HIP events (recorded by the library itself on its stream).  They only time: created with
    hipEventDisableSystemFence, a record does not write back and invalidate the caches, which would
    otherwise add several microseconds per stage boundary to the measured step."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            assert self.hip.hipEventCreateWithFlags(ctypes.byref(h), ctypes.c_uint(HIP_EVENT_DISABLE_SYSTEM_FENCE)) == 0
            self.ev.append(h)

    def elapsed_ms(self, a, b):
        f = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(f), self.ev[a], self.ev[b]) == 0
        return f.value

    def __del__(self):
        for h in getattr(self, "ev", []):
            self.hip.hipEventDestroy(h)


# After the warm-up steps, each timed workload first runs about this much more of the same work: the
# GPU's clock takes a few milliseconds of load to settle (from idle the prefill step runs 0.65-0.82 ms
# for its first ~15 steps, then 0.61-0.62 ms), and the timed steps measure the sustained rate.
SETTLE_MS = 50.0


def settle(run_one):
    """Runs `run_one()` for about SETTLE_MS of GPU time; returns how many times it ran."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_one()
    torch.cuda.synchronize()
    one_ms = max((time.perf_counter() - t0) * 1e3, 1e-3)
    n = int(math.ceil(SETTLE_MS / one_ms))
    for _ in range(n):
        run_one()
    return n + 1


def time_moe(b, steps, warmup):
    """Wall-clock ms per step over `steps` back-to-back steps (synchronized on both sides), the mean
    device time of each stage, and the median device time of a whole step (from the events the
    library records on its stream at the stage boundaries).  The warm-up steps and the settling steps
    (b.settle_steps) run before, untimed."""
    for _ in range(warmup):
        b.step()
    b.settle_steps = settle(b.step)
    ns = len(STAGES) + 1
    evs = HipEvents(steps * ns)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        b.step(evs.ev[s * ns:(s + 1) * ns])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    per_stage = np.zeros(len(STAGES))
    whole = np.zeros(steps)
    for s in range(steps):
        for j in range(len(STAGES)):
            per_stage[j] += evs.elapsed_ms(s * ns + j, s * ns + j + 1)
        whole[s] = evs.elapsed_ms(s * ns, s * ns + ns - 1)
    per_stage /= steps
    return (t1 - t0) * 1e3 / steps, per_stage, float(np.median(whole))


def time_launches(one, n, warmup):
    """Mean ms of `one(i)` over n launches queued behind a GPU-side sleep, so the host has enqueued all
    of them before the first runs: the interval between the two events is n launches back to back on
    the stream they run on, without gaps from host-side launch overhead."""
    for i in range(warmup):
        one(i)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    one(0)
    torch.cuda.synchronize()
    nsettle = int(math.ceil(SETTLE_MS / max((time.perf_counter() - t0) * 1e3, 1e-3)))
    torch.cuda._sleep(20_000_000)
    for i in range(nsettle):  # queued behind the sleep, run just before the timed launches
        one(i)
    ev[0].record()
    for i in range(n):
        one(i)
    ev[1].record()
    torch.cuda.synchronize()
    return float(ev[0].elapsed_time(ev[1])) / n


def quant_input():
    M, K = synth.QUANT_CONFIG["M"], synth.QUANT_CONFIG["K"]
    return synth.quant_matrix(M, K, cid=synth.QUANT_CONFIG["cid"])


def bench_quantize(bits, steps, warmup, rotations=4):
    """Returns the result object and the outputs of one launch (q, flat scales, tiled scales)."""
    M, K = bits.shape
    xs = [bf16_dev(bits) for _ in range(rotations)]
    qs = [torch.empty((M, K // 2), dtype=torch.uint8, device="cuda") for _ in range(rotations)]
    sfs = [torch.empty((M, K // 32), dtype=torch.uint8, device="cuda") for _ in range(rotations)]
    sts = [torch.empty(mx.tiled_scale_shape(M, K), dtype=torch.uint8, device="cuda") for _ in range(rotations)]
    L = lib()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = [[ctypes.c_void_p(t[r].data_ptr()) for t in (xs, qs, sfs, sts)] for r in range(rotations)]

    def one(i):
        a = args[i % rotations]
        check("mxfp4_quantize", L.mxfp4_quantize(a[0], M, K, K, a[1], a[2], a[3], st))
    n = max(steps, 20)
    ms = time_launches(one, n, warmup)
    nbytes = M * K * 2 + M * K // 2 + 2 * (M * K // 32)  # bf16 in, nibbles, flat + tiled scales (no padding here)
    gbs = nbytes / (ms * 1e-3) / 1e9
    res = {"workload": f"quantize bf16 {M}x{K} -> E2M1 nibbles + E8M0 flat and tiled scales", "ms": ms,
           "bytes": nbytes, "GB_s": gbs, "launches": n,
           "roofline": {"bound": "hbm", "kernel": "quantize_kernel", "achieved": gbs, "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS, "traffic": measured_traffic("quantize")}}
    torch.cuda.synchronize()
    return res, (qs[0].cpu().numpy(), sfs[0].cpu().numpy(), sts[0].cpu().numpy())


def bench_nvfp4(bits, steps, warmup, rotations=4):
    """The NVFP4 quantizer on the same matrix, with the usual per-tensor global scale (E4M3 max times
    E2M1 max over the largest magnitude)."""
    M, K = bits.shape
    xs = [bf16_dev(bits) for _ in range(rotations)]
    amax = float(xs[0].abs().max().float().item())
    gs = 448.0 * 6.0 / amax if amax > 0 else 1.0
    qs = [torch.empty((M, K // 2), dtype=torch.uint8, device="cuda") for _ in range(rotations)]
    sfs = [torch.empty((M, K // 16), dtype=torch.uint8, device="cuda") for _ in range(rotations)]
    sts = [torch.empty(mx.nvfp4_tiled_scale_shape(M, K), dtype=torch.uint8, device="cuda") for _ in range(rotations)]
    L = lib()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = [[ctypes.c_void_p(t[r].data_ptr()) for t in (xs, qs, sfs, sts)] for r in range(rotations)]

    def one(i):
        a = args[i % rotations]
        check("nvfp4_quantize", L.nvfp4_quantize(a[0], M, K, K, ctypes.c_float(gs), a[1], a[2], a[3], st))
    n = max(steps, 20)
    ms = time_launches(one, n, warmup)
    tiled = int(np.prod(mx.nvfp4_tiled_scale_shape(M, K)))
    nbytes = M * K * 2 + M * K // 2 + M * K // 16 + tiled
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": f"NVFP4 quantize bf16 {M}x{K} -> E2M1 nibbles + E4M3 flat and tiled scales (block 16)",
            "ms": ms, "bytes": nbytes, "GB_s": gbs, "frac_of_hbm": gbs / PEAK_HBM_GBS, "launches": n,
            "global_scale": gs}


def bench_linear(steps, warmup, M=8192, N=7168, K=7168):
    """The dense MXFP4-weight linear layer y = x W^T (bf16 x, MXFP4 W from N(0, 0.02) masters)."""
    g = synth.rng(181, M, N, K)
    w_bits = synth.to_bf16_bits(g.standard_normal((N, K), dtype=np.float32) * np.float32(0.02))
    x_bits = synth.to_bf16_bits(g.standard_normal((M, K), dtype=np.float32))
    wq, ws, _ = mx.quantize(bf16_dev(w_bits), flat=True, tiled=False)
    del w_bits
    layer = mx.Linear(wq, ws, None)
    del wq, ws
    xs = [bf16_dev(x_bits) for _ in range(2)]
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    n = max(steps, 20)
    ms = time_launches(lambda i: layer(xs[i % 2], y), n, warmup)
    flops = 2.0 * M * N * K
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": f"dense MXFP4-weight linear (W4A16) M={M} N={N} K={K}, bf16 in and out", "ms": ms,
            "flops": flops, "TFLOP_s": tf, "frac_of_fp4_peak": tf / PEAK_FP4_TFLOPS, "launches": n}


def moe_result(b, name, ms, stages, median_ms, iters):
    cfg = b.cfg
    return {"workload": name, "T": cfg.T, "E": cfg.E, "top_k": cfg.k, "H": cfg.H, "I": cfg.I, "bias": cfg.bias,
            "iterations": iters, "settle_steps": getattr(b, "settle_steps", 0), "ms": ms, "device_ms_median": median_ms,
            "stages_ms": {n: float(v) for n, v in zip(STAGES, stages)},
            "TFLOP_s": moe_flops(cfg) / (ms * 1e-3) / 1e12}


def expert_bytes(cfg):
    """Packed MXFP4 bytes of one expert: w13 and w2 nibbles and E8M0 scales, plus bf16 biases."""
    n = 2 * cfg.I * cfg.H // 2 + 2 * cfg.I * cfg.H // 32 + cfg.H * cfg.I // 2 + cfg.H * cfg.I // 32
    return n + (2 * (2 * cfg.I + cfg.H) if cfg.bias else 0)


def hbm_fields(res, b, extra_bytes):
    """Algorithmic bytes: the touched experts' packed weights, x, logits and y, plus `extra_bytes`."""
    cfg = b.cfg
    touched = res["expert_load"]["experts_used"]
    nbytes = touched * expert_bytes(cfg) + cfg.T * cfg.H * 4 + cfg.T * cfg.E * 4 + extra_bytes
    gbs = nbytes / (res["ms"] * 1e-3) / 1e9
    res.update({"touched_experts": touched, "algorithmic_bytes": nbytes, "GB_s": gbs, "frac_of_hbm": gbs / PEAK_HBM_GBS})


def run_tiny(args):
    cfg = synth.MOE_CONFIGS["tiny"]
    log("[bench] timing tiny MoE latency")
    b = MoeBench(cfg, rotations=2)
    ms, stages, med = time_moe(b, TINY_ITERS, args.warmup)
    res = moe_result(b, "tiny MXFP4 MoE layer (T=16, E=4, top-2, H=256, I=128, biases)", ms, stages, med, TINY_ITERS)
    res["latency_us"] = ms * 1e3
    res["expert_load"] = b.expert_load()
    return res, b.outputs()


def run_decode(args):
    cfg = synth.MOE_CONFIGS["decode"]
    log("[bench] timing decode MoE")
    b = MoeBench(cfg, rotations=2)  # two weight copies (640 MB): consecutive steps stream from HBM
    iters = max(args.steps, DECODE_ITERS)
    ms, stages, med = time_moe(b, iters, args.warmup)
    res = moe_result(b, "decode-shaped MXFP4 MoE layer (T=64, E=128, top-8, H=2048, I=768, biases)", ms, stages, med,
                     iters)
    res["expert_load"] = b.expert_load()
    hbm_fields(res, b, 0)
    return res, b.outputs()


def run_large(args):
    cfg = synth.MOE_CONFIGS["large"]
    log(f"[bench] building large-expert workload T={cfg.T} E={cfg.E} k={cfg.k} H={cfg.H} I={cfg.I}")
    b = MoeBench(cfg, rotations=2, weight_copies=1)  # 9 GB of weights: nothing survives in the cache
    log("[bench] timing large-expert MoE")
    ms, stages, med = time_moe(b, args.steps, args.warmup)
    res = moe_result(b, "large-expert MXFP4 MoE layer (T=4096, E=384, top-8, H=7168, I=2048, Zipf(1.2) routing)",
                     ms, stages, med, args.steps)
    res["expert_load"] = b.expert_load()
    # plus the SwiGLU activation written and read once in bf16
    hbm_fields(res, b, cfg.T * cfg.k * cfg.I * 4)
    res["frac_of_fp4_peak"] = res["TFLOP_s"] / PEAK_FP4_TFLOPS
    return res, b.outputs()


def run_prefill(args):
    cfg = synth.MOE_CONFIGS["prefill"]
    log(f"[bench] building prefill workload T={cfg.T} E={cfg.E} k={cfg.k} H={cfg.H} I={cfg.I}")
    b = MoeBench(cfg, rotations=2)
    log("[bench] timing prefill MoE")
    ms, stages, med = time_moe(b, args.steps, args.warmup)
    b.prefill_settle_steps = b.settle_steps
    o = b.outputs()
    load = b.expert_load()
    variants = {}
    if not args.no_variants:
        for name, act in (("mxfp8_activations", mx.ACT_MXFP8), ("mxfp4_activations", mx.ACT_MXFP4)):
            log(f"[bench] timing prefill MoE, {name}")
            b.act = act
            vms, vst, vmed = time_moe(b, args.steps, args.warmup)
            variants[name] = moe_result(b, f"prefill-shaped MXFP4 MoE layer, {name.replace('_', ' ')}", vms, vst, vmed,
                                        args.steps)
            variants[name]["frac_of_fp4_peak"] = variants[name]["TFLOP_s"] / PEAK_FP4_TFLOPS
        b.act = mx.ACT_BF16
    return b, ms, stages, med, o, load, variants


def moe_parity(y_gpu, y_ref, rows=None):
    """max |err| / rms(y_ref) and the number of elements outside |err| <= 2e-2 * rms + 1e-3 (rms over
    the compared rows)."""
    ref = y_ref if rows is None else y_ref[rows]
    got = y_gpu if rows is None else y_gpu[rows]
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = np.abs(got - ref)
    return {"max_err_over_rms": float(err.max() / rms) if rms > 0 else float(err.max()),
            "mismatches": int(np.count_nonzero(err > RTOL_RMS * rms + ATOL)), "compared": int(err.size),
            "tolerance": "|y - y_ref| <= 2e-2 * rms(y_ref) + 1e-3"}


def cpu_leg(cpu, outputs, out):
    """The oracle, untuned, timed on the host cores: every token of the tiny, decode and prefill
    workloads, a sample of the large-expert workload, the whole quantize matrix.  Its results also give
    the parity figures of the library's outputs from the same run.  Quantizing the bf16 masters for the
    oracle is input preparation and is not timed."""
    from oracle import moe as M
    from oracle import quant as Q
    from oracle.route import route_ref
    from tests.gpu_common import LazyExperts

    def prep_experts(cfg, tokens):
        ids, _ = route_ref(outputs[cfg.name]["logits"], cfg.k)
        used = np.unique(ids[tokens])
        w13, w2 = LazyExperts(cfg, "w13"), LazyExperts(cfg, "w2")
        with ThreadPoolExecutor(workers()) as ex:
            list(ex.map(lambda e: (w13.get(e), w2.get(e)), used))
        b13, b2 = synth.moe_biases(cfg)
        return w13, w2, b13, b2, len(used)

    def time_oracle(cfg, tokens, repeats):
        w13, w2, b13, b2, nused = prep_experts(cfg, tokens)
        o = outputs[cfg.name]
        times, y = [], None
        for _ in range(repeats):
            t0 = time.perf_counter()
            y = M.moe_ref(o["x_bits"], o["logits"], cfg.k, w13.q, w13.s, w2.q, w2.s, b13, b2, renormalize=cfg.renormalize,
                          tokens=tokens)[0]
            times.append(time.perf_counter() - t0)
        dt = float(np.median(times))
        flops = 2.0 * len(tokens) * cfg.k * 3 * cfg.H * cfg.I
        base = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cpu["cores"], "blas_threads": cpu["blas_threads"],
                "cpu_model": cpu["model"], "kind": "oracle", "seconds": dt, "repeats": repeats}
        return base, y, nused

    for name, key in (("tiny", "tiny"), ("decode", "decode"), ("prefill", None), ("large", "large")):
        if name not in outputs:
            continue
        cfg = synth.MOE_CONFIGS[name]
        if name == "large":
            tokens = np.arange(LARGE_SAMPLE_TOKENS)
            repeats = 1
        else:
            tokens = np.arange(cfg.T)
            repeats = 1 if name == "prefill" else 3
        log(f"[bench] timing the CPU oracle on the {name} workload ({len(tokens)} tokens)")
        base, y_ref, nused = time_oracle(cfg, tokens, repeats)
        what = "all" if len(tokens) == cfg.T else "the first"
        base["sample"] = (f"{what} {len(tokens)} of {cfg.T} tokens ({nused} experts used, dequantized in fp64); "
                          "weights pre-quantized outside the timed region")
        par = moe_parity(outputs[name]["y"], y_ref, None if len(tokens) == cfg.T else tokens)
        if key is None:
            out["cpu_baseline"] = base
            out["parity"] = par
        else:
            out[key]["cpu_baseline"] = base
            out[key]["parity"] = par

    if "quantize" in outputs:
        log("[bench] timing the CPU oracle on the quantize matrix")
        bits = outputs["quantize"]["bits"]
        Mq, K = bits.shape
        times = []
        for _ in range(3):
            t0 = time.perf_counter()
            q, s = Q.quantize_ref(bits)
            st = Q.tile_scales(s)
            times.append(time.perf_counter() - t0)
        dt = float(np.median(times))
        nbytes = Mq * K * 2 + Mq * K // 2 + 2 * Mq * K // 32
        out["quantize"]["cpu_baseline"] = {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": cpu["cores"],
                                           "cpu_model": cpu["model"], "kind": "oracle", "seconds": dt, "repeats": 3,
                                           "sample": f"all {Mq} rows of the quantize matrix"}
        gq, gsf, gst = outputs["quantize"]["gpu"]
        # saturation: elements whose magnitude over the block scale exceeds E2M1's largest value 6
        mag = np.abs(Q.bf16_to_f64(bits)).reshape(Mq, K // 32, 32)
        ratio = mag * np.exp2(127.0 - s.astype(np.float64))[:, :, None]
        sat = ratio > 6.0
        nonzero = mag > 0
        out["quantize"]["parity"] = {
            "nibble_byte_mismatches": int(np.count_nonzero(gq != q)), "flat_scale_mismatches": int(np.count_nonzero(gsf != s)),
            "tiled_scale_mismatches": int(np.count_nonzero(gst != st)), "compared_bytes": int(q.size + s.size + st.size),
            "saturated_element_fraction": float(sat.sum() / sat.size),
            "blocks_with_a_saturated_element": int(np.count_nonzero(sat.any(axis=2))),
            "blocks_saturated_whole": int(np.count_nonzero((sat | ~nonzero).all(axis=2) & nonzero.any(axis=2))),
            "blocks": int(Mq * K // 32)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--only", choices=["prefill", "tiny", "decode", "quantize", "large", "nvfp4", "linear"], default=None,
                    help="time one workload only (for profiler runs); the JSON line then holds that workload")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this library has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "needs a GPU"
    torch.cuda.set_device(0)
    if args.only is not None:
        args.no_cpu_baseline = True
        args.no_variants = True
        if args.only != "prefill":
            out = {"metric": METRIC, "only": args.only}
            if args.only in ("tiny", "decode", "large"):
                out[args.only] = {"tiny": run_tiny, "decode": run_decode, "large": run_large}[args.only](args)[0]
            elif args.only == "quantize":
                out["quantize"] = bench_quantize(quant_input(), args.steps, args.warmup)[0]
            elif args.only == "nvfp4":
                out["nvfp4"] = bench_nvfp4(quant_input(), args.steps, args.warmup)
            else:
                out["linear"] = bench_linear(args.steps, args.warmup)
            print(json.dumps(out), flush=True)
            return

    cpu = host_cpu()
    outputs = {}
    cfg = synth.MOE_CONFIGS["prefill"]
    b, ms, stages, med, outputs["prefill"], load, variants = run_prefill(args)
    flops = moe_flops(cfg)
    value = flops / (ms * 1e-3) / 1e12
    P = cfg.T * cfg.k
    g1_flops = 2.0 * P * cfg.H * 2 * cfg.I
    g2_flops = 2.0 * P * cfg.I * cfg.H
    g1_ms, g2_ms = stages[STAGES.index("gemm1_swiglu")], stages[STAGES.index("gemm2_weighted")]
    # the dominant kernel: algorithmic flops of the first GEMM per launch over its measured launch time
    # (HIP events the library records on its own stream around the launch).  The MFMA issues every
    # product once per activation term, so the matrix cores execute three times the algorithmic flops.
    g1_tf = g1_flops / (g1_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": "grouped_gemm_kernel<G1=true> (first grouped GEMM + SwiGLU)",
                "achieved": g1_tf, "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s", "frac": g1_tf / PEAK_FP4_TFLOPS,
                "traffic": measured_traffic("gemm"), "flops_per_launch": g1_flops, "avg_launch_ms": g1_ms,
                "mfma_issued_frac": ACT_TERMS * g1_tf / PEAK_FP4_TFLOPS}
    out = {
        "metric": METRIC,
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": DTYPE, "data": "synthetic",
        "config": {"workload": "prefill-shaped MXFP4 MoE layer, bf16 tokens", "T": cfg.T, "E": cfg.E, "top_k": cfg.k,
                   "H": cfg.H, "I": cfg.I, "bias": cfg.bias, "parallelism": "single GPU"},
        "roofline": roofline,
        "settle_steps": b.prefill_settle_steps,
        "timing": f"{args.steps} steps timed after {args.warmup} warm-up steps and {b.prefill_settle_steps} settling steps "
                  f"(about {SETTLE_MS:g} ms of the same work, while the GPU clock settles under load)",
        "device_ms_median": med,
        "stages_ms": {n: float(v) for n, v in zip(STAGES, stages)},
        "layer_frac_of_fp4_peak": value / PEAK_FP4_TFLOPS,
        "stage_kernels": dict(zip(STAGES, STAGE_KERNELS)),
        "gemm2": {"kernel": "grouped_gemm_kernel<G1=false>", "achieved_TFLOP_s": g2_flops / (g2_ms * 1e-3) / 1e12,
                  "frac": g2_flops / (g2_ms * 1e-3) / 1e12 / PEAK_FP4_TFLOPS, "avg_launch_ms": g2_ms},
        "expert_load": load,
        "host_cpu": cpu,
    }
    if variants:
        out["variants"] = variants
    del b
    torch.cuda.empty_cache()
    if args.only == "prefill":
        print(json.dumps(out), flush=True)
        return

    bits = quant_input()
    log("[bench] timing quantize")
    out["quantize"], gq = bench_quantize(bits, args.steps, args.warmup)
    outputs["quantize"] = {"bits": bits, "gpu": gq}
    torch.cuda.empty_cache()
    log("[bench] timing NVFP4 quantize")
    out["nvfp4"] = bench_nvfp4(bits, args.steps, args.warmup)
    torch.cuda.empty_cache()
    log("[bench] timing the dense MXFP4 linear layer")
    out["linear"] = bench_linear(args.steps, args.warmup)
    torch.cuda.empty_cache()

    for name, fn in (("tiny", run_tiny), ("decode", run_decode), ("large", run_large)):
        out[name], outputs[name] = fn(args)
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        cpu_leg(cpu, outputs, out)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
