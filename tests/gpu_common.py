"""Helpers shared by the GPU parity tests, the smoke check and the benchmark: moving the seeded inputs
to the device, building the HIP path's weights from the bf16 masters, and the oracle-side weights of
the same masters (quantized lazily, one expert at a time)."""

import collections
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import mixed_precision_moe_amd as mx
from mixed_precision_moe_amd import synth

RTOL_RMS, ATOL = 2e-2, 1e-3  # |y - y_ref| <= 2e-2 * rms(y_ref) + 1e-3


def device():
    assert torch.cuda.is_available(), "a GPU is required"
    return torch.device("cuda:0")


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device()).view(torch.bfloat16)


def bf16_host_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_host_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def workers():
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, n))


def ordered_prefetch(fn, items, window=None):
    """Yield fn(item) in order, computing up to `window` items ahead on a thread pool."""
    window = window or workers()
    with ThreadPoolExecutor(max_workers=window) as ex:
        q = collections.deque()
        it = iter(items)
        for _ in range(window):
            try:
                q.append(ex.submit(fn, next(it)))
            except StopIteration:
                break
        while q:
            r = q.popleft().result()
            try:
                q.append(ex.submit(fn, next(it)))
            except StopIteration:
                pass
            yield r


def gpu_standard_weights(cfg):
    """Quantize every expert's bf16 masters on the GPU with the library's quantizer.
    Returns device tensors (w13_q, w13_s, w2_q, w2_s, b13, b2) in the standard checkpoint layout."""
    dev = device()
    E, H, I = cfg.E, cfg.H, cfg.I
    w13_q = torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device=dev)
    w13_s = torch.empty((E, 2 * I, H // 32), dtype=torch.uint8, device=dev)
    w2_q = torch.empty((E, H, I // 2), dtype=torch.uint8, device=dev)
    w2_s = torch.empty((E, H, I // 32), dtype=torch.uint8, device=dev)
    for e, (m13, m2) in enumerate(ordered_prefetch(lambda e: synth.moe_master_expert(cfg, e), range(E))):
        q, s, _ = mx.quantize(bf16_dev(m13), flat=True, tiled=False)
        w13_q[e].copy_(q)
        w13_s[e].copy_(s)
        q, s, _ = mx.quantize(bf16_dev(m2), flat=True, tiled=False)
        w2_q[e].copy_(q)
        w2_s[e].copy_(s)
    b13, b2 = synth.moe_biases(cfg)
    if b13 is not None:
        b13, b2 = bf16_dev(b13), bf16_dev(b2)
    torch.cuda.synchronize()
    return w13_q, w13_s, w2_q, w2_s, b13, b2


class OracleExperts:
    """Oracle-side expert weights held in memory: q and s index like stacked [E, ...] arrays."""

    def __init__(self, E, rows, K):
        self.qs = [None] * E
        self.ss = [None] * E
        self.q = _View(self, 0, (E, rows, K // 2))
        self.s = _View(self, 1, (E, rows, K // 32))

    def get(self, e):
        return self.qs[e], self.ss[e]


def prepared_weights(cfg):
    """Both sides' weights from one generation of the bf16 masters: the library quantizes them on the
    GPU (device tensors in the standard layout, as gpu_standard_weights), the oracle quantizes the same
    masters itself on worker threads.  Returns (device tensors, oracle w13, oracle w2)."""
    from oracle import quant as Q
    dev = device()
    E, H, I = cfg.E, cfg.H, cfg.I
    w13_q = torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device=dev)
    w13_s = torch.empty((E, 2 * I, H // 32), dtype=torch.uint8, device=dev)
    w2_q = torch.empty((E, H, I // 2), dtype=torch.uint8, device=dev)
    w2_s = torch.empty((E, H, I // 32), dtype=torch.uint8, device=dev)
    o13, o2 = OracleExperts(E, 2 * I, H), OracleExperts(E, H, I)

    def prep(e):
        m13, m2 = synth.moe_master_expert(cfg, e)
        return m13, m2, Q.quantize_ref(m13), Q.quantize_ref(m2)

    for e, (m13, m2, r13, r2) in enumerate(ordered_prefetch(prep, range(E))):
        q, s, _ = mx.quantize(bf16_dev(m13), flat=True, tiled=False)
        w13_q[e].copy_(q)
        w13_s[e].copy_(s)
        q, s, _ = mx.quantize(bf16_dev(m2), flat=True, tiled=False)
        w2_q[e].copy_(q)
        w2_s[e].copy_(s)
        o13.qs[e], o13.ss[e] = r13
        o2.qs[e], o2.ss[e] = r2
    b13, b2 = synth.moe_biases(cfg)
    if b13 is not None:
        b13, b2 = bf16_dev(b13), bf16_dev(b2)
    torch.cuda.synchronize()
    return (w13_q, w13_s, w2_q, w2_s, b13, b2), o13, o2


def oracle_moe_threaded(x_bits, logits, k, w13, w2, b13, b2, renormalize=True, tokens=None, act="bf16",
                        with_slack=False):
    """The oracle's MoE layer with its experts spread over worker threads (one BLAS thread each): y is
    the sum of the results over a partition of the experts (and so is the near-tie slack of the
    quantized-activation variants, returned as well when with_slack)."""
    from oracle import moe as M
    E = w13.q.shape[0]
    n = workers()
    parts = [list(range(i, E, n)) for i in range(n)]
    T, H = x_bits.shape

    def part(ex_ids):
        sl = np.zeros((T, H)) if with_slack else None
        y = M.moe_ref(x_bits, logits, k, w13.q, w13.s, w2.q, w2.s, b13, b2, renormalize=renormalize, tokens=tokens,
                      experts=ex_ids, act=act, slack=sl)[0]
        return y, sl

    from threadpoolctl import threadpool_limits
    with threadpool_limits(1), ThreadPoolExecutor(max_workers=n) as ex:
        res = list(ex.map(part, parts))
    y = sum((r[0] for r in res[1:]), res[0][0])
    if not with_slack:
        return y
    return y, sum((r[1] for r in res[1:]), res[0][1])


class LazyExperts:
    """Oracle-side expert weights: the same bf16 masters quantized by the oracle, one expert at a time
    on first use.  Indexing yields (q, s) arrays of one expert, like slicing a stacked [E, ...] array."""

    def __init__(self, cfg, which):
        from oracle import quant as Q
        self._Q, self.cfg, self.which = Q, cfg, which
        rows, K = (2 * cfg.I, cfg.H) if which == "w13" else (cfg.H, cfg.I)
        self._cache = {}
        self.q = _View(self, 0, (cfg.E, rows, K // 2))
        self.s = _View(self, 1, (cfg.E, rows, K // 32))

    def get(self, e):
        if e not in self._cache:
            m13, m2 = synth.moe_master_expert(self.cfg, e)
            self._cache[e] = self._Q.quantize_ref(m13 if self.which == "w13" else m2)
        return self._cache[e]


class _View:
    def __init__(self, owner, idx, shape):
        self.owner, self.idx, self.shape = owner, idx, shape

    def __getitem__(self, e):
        return self.owner.get(int(e))[self.idx]


def assert_moe_close(y_gpu, y_ref, rows=None, what="", slack=None):
    """Elementwise |y - y_ref| <= 2e-2 * rms(y_ref) + 1e-3 (+ slack, the oracle's bound for near-tie
    quantization decisions of the quantized-activation variants) on `rows` (all rows if None); rms is
    taken over the compared rows.  Returns (max |err| / rms, number of violations)."""
    ref = y_ref if rows is None else y_ref[rows]
    got = y_gpu if rows is None else y_gpu[rows]
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = np.abs(got - ref)
    bound = RTOL_RMS * rms + ATOL
    if slack is not None:
        bound = bound + (slack if rows is None else slack[rows])
    bad = int(np.count_nonzero(err > bound))
    ratio = float(err.max() / rms) if rms > 0 else float(err.max())
    assert bad == 0, f"{what}: {bad} of {err.size} elements outside tolerance (max err/rms {ratio:.4g})"
    return ratio, bad
