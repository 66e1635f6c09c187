"""Oracle: the MXFP4-weight x BF16-activation MoE layer, evaluated in float64.

Test infrastructure only (see the package docstring).

Per token t with selected experts e_j and weights w_j (route_ref):
    h   = x_t . W13_e^T + b13_e          W13_e = dequant(w13_q[e], w13_s[e]), rows [w1; w3]
    a   = silu(h[:I]) * h[I:]            silu(g) = g / (1 + exp(-g))
    o   = a . W2_e^T + b2_e              W2_e  = dequant(w2_q[e], w2_s[e])
    y_t = sum_j w_j * o_j
[DEF: grouped w13 GEMM, SwiGLU as silu(w1 half) * (w3 half), grouped w2 GEMM, weighted combine;
 P2 Implementation breakdown item 2: the checkpoint's fused gate/up is [w1; w3]]
Reading: b13 is added before the activation and b2 to each expert's output before weighting.
"""

import math
import struct

import numpy as np

from . import quant as Q
from .quant import bf16_to_f64, dequant_ref, E2M1_MAGNITUDES
from .route import route_ref

ACT_FORMATS = ("bf16", "mxfp8", "mxfp4")
"""Activation formats of the layer: bf16 activations (the two GEMMs take the activations as they are),
or both GEMM inputs quantized per 32-element block with an E8M0 scale, to MXFP8 (E4M3 elements; the
MXFP8-activation variant [P2 Implementation breakdown item 3]) or to MXFP4 (E2M1 elements, the same
rule as the weights; the experts-quant step [P3 Implementation breakdown item 3]).  Reading: the layer
input x and the SwiGLU output are the activations quantized (the pages name the variants, not the
points); the SwiGLU output is rounded to binary32 first, the precision in which the kernel decides."""

AMBIGUITY_REL = 2.0 ** -16
"""Relative window around a rounding decision of the quantized SwiGLU output within which the
kernel's binary32 arithmetic (other summation order, hardware exp) may decide the other way: about
ten times the relative difference between a binary32 SwiGLU computed that way and the float64 one
rounded to binary32."""


def silu(g):
    return g / (1.0 + np.exp(-g))


def quantize_activation(vals32, act):
    """Dequantized float64 values of binary32 activations [n, K] under format `act` (mxfp8 or mxfp4)."""
    if act == "mxfp8":
        c, s = Q.mxfp8_quantize_values_ref(vals32)
        return Q.mxfp8_dequant_ref(c, s)
    c, s = Q.quantize_values_ref(vals32)
    return Q.dequant_codes_ref(c, s)


def activation_ambiguity(vals32, act, rel=AMBIGUITY_REL):
    """Per element, the largest change of its dequantized value when the block's values move by up to
    rel of themselves plus rel / 64 of the block maximum, all up or all down (a rounding midpoint or
    the scale's round-up threshold crossed).  0 where every decision is clear of the window."""
    v = np.asarray(vals32, dtype=np.float64)
    base = quantize_activation(vals32, act)
    n, K = v.shape
    bmax = np.repeat(np.abs(v.reshape(n, K // 32, 32)).max(axis=-1), 32, axis=-1)
    d = np.zeros_like(v)
    for sgn in (-1.0, 1.0):
        p = v + sgn * (rel * np.abs(v) + rel / 64 * bmax) * np.sign(v)
        d = np.maximum(d, np.abs(quantize_activation(p.astype(np.float32), act) - base))
    return d


def moe_ref(x_bits, logits, k, w13_q, w13_s, w2_q, w2_s, b13_bits=None, b2_bits=None,
            renormalize=True, tokens=None, experts=None, act="bf16", slack=None):
    """Vectorized float64 MoE layer, one expert at a time (bounded memory for large E*I*H).

    x_bits uint16 [T, H] bf16; logits float32 [T, E]; w13_q uint8 [E, 2I, H/2]; w13_s uint8
    [E, 2I, H/32]; w2_q uint8 [E, H, I/2]; w2_s uint8 [E, H, I/32]; biases bf16 bit patterns
    [E, 2I] / [E, H] or None.  ``tokens``: optional index array; only those rows of y are computed
    (the others stay 0), which lets large configurations be checked on a sample of tokens.
    ``experts``: optional expert ids; only their terms w_j * o_j are summed into y, so the layer is
    the sum of the results over any partition of the experts (the sum over j has no prescribed order).
    ``act``: one of ACT_FORMATS.  For mxfp8 / mxfp4 the rows of x are quantized before the first
    product and the SwiGLU output, rounded to binary32, before the second; ``slack`` (float64 [T, H],
    optional) then receives, added per token, w_j * sum_i amb_i * |W2[:, i]| with amb the
    activation_ambiguity of that expert's SwiGLU output: a bound on how far a result whose near-tie
    decisions went the other way can lie from y.
    Returns (y float64 [T, H], ids int32 [T, k], w float64 [T, k]).
    """
    if act not in ACT_FORMATS:
        raise ValueError(f"unknown activation format {act!r}")
    ids, w = route_ref(logits, k, renormalize)
    x = bf16_to_f64(x_bits)
    T, H = x.shape
    E = w13_q.shape[0]
    I = w2_q.shape[2] * 2
    rows = np.arange(T) if tokens is None else np.unique(np.asarray(tokens))
    y = np.zeros((T, H))
    sub_ids = ids[rows]
    for e in (range(E) if experts is None else experts):
        r_idx, j_idx = np.nonzero(sub_ids == e)
        if r_idx.size == 0:
            continue
        t_idx = rows[r_idx]
        W13 = dequant_ref(w13_q[e], w13_s[e])
        W2 = dequant_ref(w2_q[e], w2_s[e])
        xe = x[t_idx]
        if act != "bf16":
            xe = quantize_activation(xe.astype(np.float32), act)  # bf16 values: exact in binary32
        h = xe @ W13.T
        if b13_bits is not None:
            h = h + bf16_to_f64(b13_bits[e])
        a = silu(h[:, :I]) * h[:, I:]
        if act != "bf16":
            a32 = a.astype(np.float32)
            if slack is not None:
                amb = activation_ambiguity(a32, act)
                np.add.at(slack, t_idx, w[t_idx, j_idx][:, None] * (amb @ np.abs(W2).T))
            a = quantize_activation(a32, act)
        o = a @ W2.T
        if b2_bits is not None:
            o = o + bf16_to_f64(b2_bits[e])
        np.add.at(y, t_idx, w[t_idx, j_idx][:, None] * o)
    return y, ids, w


def _decode_weight(qrow, srow, kk):
    """Value of element kk of one packed weight row, decoded one nibble at a time."""
    byte = int(qrow[kk // 2])
    nib = (byte >> 4) if (kk & 1) else (byte & 0xF)
    mag = float(E2M1_MAGNITUDES[nib & 7])
    return (-mag if nib & 8 else mag) * 2.0 ** (int(srow[kk // 32]) - 127)


def _scalar_quantize_block(vals, act):
    """One block of 32 Python floats (binary32 values) -> their dequantized values, one at a time:
    the scale from math.frexp of the block maximum (round up at a significand of 1.75, minus the
    element format's largest exponent: 2 for E2M1, 8 for E4M3), each element the nearest magnitude of
    the format's table by a linear search (the even code on a tie)."""
    table = [float(v) for v in (Q.E4M3_MAGNITUDES if act == "mxfp8" else E2M1_MAGNITUDES)]
    emax = 8 if act == "mxfp8" else 2
    amax = max(abs(v) for v in vals)
    if amax > 0:
        m, ex = math.frexp(amax)
        e = min(max((ex - 1) + 127 + (1 if 2 * m >= 1.75 else 0) - emax, 0), 254)
    else:
        e = 0
    scale = 2.0 ** (e - 127)
    out = []
    for v in vals:
        t = abs(v) / scale
        best = 0
        for c in range(len(table)):
            dc, db = abs(t - table[c]), abs(t - table[best])
            if dc < db or (dc == db and c % 2 == 0 and best % 2 == 1):
                best = c
        out.append(math.copysign(table[best] * scale, v))
    return out


def _f32(v):
    return struct.unpack("<f", struct.pack("<f", v))[0]


def moe_bruteforce(x_bits, logits, k, w13_q, w13_s, w2_q, w2_s, b13_bits=None, b2_bits=None,
                   renormalize=True, act="bf16"):
    """Literal per-token, per-expert, per-output-scalar loop in pure Python (tiny shapes only).

    Routing is re-done by a full Python sort with key (-logit, expert), weights with math.exp, and
    every weight is decoded from its own nibble and scale byte; dot products use math.fsum.  With a
    quantized activation format, x and the SwiGLU output (rounded to binary32 with struct) are
    quantized block by block by _scalar_quantize_block.
    """
    T, H = x_bits.shape
    E = w13_q.shape[0]
    I = w2_q.shape[2] * 2
    x = [[float(v) for v in bf16_to_f64(x_bits[t])] for t in range(T)]
    y = np.zeros((T, H))
    for t in range(T):
        lt = [float(v) for v in np.asarray(logits[t], dtype=np.float32)]
        order = sorted(range(E), key=lambda e: (-lt[e], e))[:k]
        lmax = max(lt)
        ex = [math.exp(lt[e] - lmax) for e in range(E)]
        denom = math.fsum(ex[e] for e in order) if renormalize else math.fsum(ex)
        xt = x[t]
        if act != "bf16":
            xt = [v for b0 in range(0, H, 32) for v in _scalar_quantize_block(xt[b0:b0 + 32], act)]
        for e in order:
            we = ex[e] / denom
            h = []
            for n in range(2 * I):
                s = math.fsum(xt[kk] * _decode_weight(w13_q[e][n], w13_s[e][n], kk) for kk in range(H))
                if b13_bits is not None:
                    s += float(bf16_to_f64(b13_bits[e][n]))
                h.append(s)
            a = [h[i] / (1.0 + math.exp(-h[i])) * h[I + i] for i in range(I)]
            if act != "bf16":
                a = [_f32(v) for v in a]
                a = [v for b0 in range(0, I, 32) for v in _scalar_quantize_block(a[b0:b0 + 32], act)]
            for m in range(H):
                o = math.fsum(a[i] * _decode_weight(w2_q[e][m], w2_s[e][m], i) for i in range(I))
                if b2_bits is not None:
                    o += float(bf16_to_f64(b2_bits[e][m]))
                y[t, m] += we * o
    return y
