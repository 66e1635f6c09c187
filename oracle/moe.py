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

import numpy as np

from .quant import bf16_to_f64, dequant_ref, E2M1_MAGNITUDES
from .route import route_ref


def silu(g):
    return g / (1.0 + np.exp(-g))


def moe_ref(x_bits, logits, k, w13_q, w13_s, w2_q, w2_s, b13_bits=None, b2_bits=None,
            renormalize=True, tokens=None, experts=None):
    """Vectorized float64 MoE layer, one expert at a time (bounded memory for large E*I*H).

    x_bits uint16 [T, H] bf16; logits float32 [T, E]; w13_q uint8 [E, 2I, H/2]; w13_s uint8
    [E, 2I, H/32]; w2_q uint8 [E, H, I/2]; w2_s uint8 [E, H, I/32]; biases bf16 bit patterns
    [E, 2I] / [E, H] or None.  ``tokens``: optional index array; only those rows of y are computed
    (the others stay 0), which lets large configurations be checked on a sample of tokens.
    ``experts``: optional expert ids; only their terms w_j * o_j are summed into y, so the layer is
    the sum of the results over any partition of the experts (the sum over j has no prescribed order).
    Returns (y float64 [T, H], ids int32 [T, k], w float64 [T, k]).
    """
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
        h = x[t_idx] @ W13.T
        if b13_bits is not None:
            h = h + bf16_to_f64(b13_bits[e])
        a = silu(h[:, :I]) * h[:, I:]
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


def moe_bruteforce(x_bits, logits, k, w13_q, w13_s, w2_q, w2_s, b13_bits=None, b2_bits=None,
                   renormalize=True):
    """Literal per-token, per-expert, per-output-scalar loop in pure Python (tiny shapes only).

    Routing is re-done by a full Python sort with key (-logit, expert), weights with math.exp, and
    every weight is decoded from its own nibble and scale byte; dot products use math.fsum.
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
        for e in order:
            we = ex[e] / denom
            h = []
            for n in range(2 * I):
                s = math.fsum(x[t][kk] * _decode_weight(w13_q[e][n], w13_s[e][n], kk) for kk in range(H))
                if b13_bits is not None:
                    s += float(bf16_to_f64(b13_bits[e][n]))
                h.append(s)
            a = [h[i] / (1.0 + math.exp(-h[i])) * h[I + i] for i in range(I)]
            for m in range(H):
                o = math.fsum(a[i] * _decode_weight(w2_q[e][m], w2_s[e][m], i) for i in range(I))
                if b2_bits is not None:
                    o += float(bf16_to_f64(b2_bits[e][m]))
                y[t, m] += we * o
    return y
