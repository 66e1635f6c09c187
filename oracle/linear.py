"""Oracle: the dense MXFP4-weight x BF16-activation linear layer, evaluated in float64.

Test infrastructure only (see the package docstring).

    y = x . W^T + b,   W = dequant(w_q, w_s)   (MXFP4 rows [N, K/2] and E8M0 scales [N, K/32])

[P3 Implementation breakdown item 2: the MXFP4 linear path (apply_weights, made contiguous before its
activation is quantized); DEF: the linear layer with MXFP4 weights and 16-bit activations (W4A16), a
MoE layer of one expert without routing or activation function]
Reading: the bias, when present, is added after the product.
"""

import numpy as np

from .quant import bf16_to_f64, dequant_ref, E2M1_MAGNITUDES


def linear_ref(x_bits, w_q, w_s, b_bits=None):
    """x_bits uint16 [M, K] bf16; w_q uint8 [N, K/2]; w_s uint8 [N, K/32]; b_bits uint16 [N] bf16 or
    None.  Returns y float64 [M, N]."""
    y = bf16_to_f64(x_bits) @ dequant_ref(w_q, w_s).T
    if b_bits is not None:
        y = y + bf16_to_f64(b_bits)[None, :]
    return y


def linear_bruteforce(x_bits, w_q, w_s, b_bits=None):
    """Per output scalar, in pure Python: every weight decoded from its own nibble and scale byte,
    the dot product with math.fsum (tiny shapes only)."""
    import math
    M, K = x_bits.shape
    N = w_q.shape[0]
    x = bf16_to_f64(x_bits)
    y = np.zeros((M, N))
    for n in range(N):
        row = []
        for k in range(K):
            byte = int(w_q[n, k // 2])
            nib = (byte >> 4) if (k & 1) else (byte & 0xF)
            mag = float(E2M1_MAGNITUDES[nib & 7])
            row.append((-mag if nib & 8 else mag) * 2.0 ** (int(w_s[n, k // 32]) - 127))
        for m in range(M):
            s = math.fsum(float(x[m, k]) * row[k] for k in range(K))
            if b_bits is not None:
                s += float(bf16_to_f64(b_bits[n]))
            y[m, n] = s
    return y
