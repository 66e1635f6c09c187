"""Input construction for the exhaustive element test of the quantizer.

Every finite bf16 pattern is placed under every E8M0 exponent e in [0, 253] that it can meet: each
32-element block starts with the largest bf16 magnitude whose block scale is e, and its other 31
elements are patterns no larger than that magnitude, so the block's scale is e and each pattern is
encoded under it.  Test-only; used by the oracle pin and by the GPU parity test alike.
"""

import numpy as np


def amax_for_scale(e):
    """Largest bf16 magnitude pattern whose E8M0 scale is e: the block maximum m gets scale e for
    m in [1.75 * 2**(e-126), 1.75 * 2**(e-125)); the largest bf16 below the upper end has biased
    exponent e + 2 and mantissa 0x5F (1.7421875); e = 253 takes the largest finite bf16."""
    if e == 253:
        return 0x7F7F
    return ((e + 2) << 7) | 0x5F


def exhaustive_blocks(e):
    """uint16 [n_blocks, 32] for scale e: column 0 is amax_for_scale(e), the rest are all finite
    patterns (both signs) with magnitude <= it, in increasing order, the last block padded with 0."""
    top = amax_for_scale(e)
    mags = np.arange(0, top + 1, dtype=np.uint32)
    pats = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
    nb = (pats.size + 30) // 31
    body = np.zeros(nb * 31, dtype=np.uint16)
    body[: pats.size] = pats
    out = np.empty((nb, 32), dtype=np.uint16)
    out[:, 0] = top
    out[:, 1:] = body.reshape(nb, 31)
    return out


def exhaustive_matrix(es=range(254)):
    """Stack exhaustive_blocks for several exponents; returns (bits [rows, 32], expected_e [rows])."""
    parts, ees = [], []
    for e in es:
        b = exhaustive_blocks(e)
        parts.append(b)
        ees.append(np.full(b.shape[0], e, dtype=np.uint8))
    return np.concatenate(parts), np.concatenate(ees)
