"""Oracle: the checkpoint conversions of the MoE weight set.

Test infrastructure only (see the package docstring).

The standard MXFP4 checkpoint stores the fused gate/up projection as w13 = [w1; w3] along the row
dimension (dim 1 of [E, 2I, ...]), w2 as [E, H, I/2], E8M0 scales as uint8 and optional biases.
[P2 Implementation breakdown, item 2; Key source snippets, the conversion branch for the FlashInfer
CUTLASS backends]
"""

import numpy as np

from .quant import tile_scales


def swap_w13_w31(w13):
    """[w1; w3] -> [w3; w1]: swap the two halves of dim 1 (rows of the fused gate/up tensor).

    Applies unchanged to the packed weights [E, 2I, H/2] and to their scales [E, 2I, H/32].
    [P2 Implementation breakdown, item 2; the page's test expects the second half of the rows first]
    """
    w13 = np.asarray(w13)
    if w13.shape[1] % 2:
        raise ValueError("dim 1 of w13 must be even")
    half = w13.shape[1] // 2
    return np.concatenate([w13[:, half:], w13[:, :half]], axis=1)


def swap_b13_b31(b13):
    """The fused bias [E, 2I] is split in two along its last dimension and the halves are exchanged.
    [P2 Key source snippets, chunk into (b1, b3) and concatenate (b3, b1)]"""
    b13 = np.asarray(b13)
    half = b13.shape[-1] // 2
    return np.concatenate([b13[..., half:], b13[..., :half]], axis=-1)


def f32_to_bf16_bits(x):
    """binary32 -> bf16 bit pattern, round to nearest, ties to even (NaN/Inf out of contract).

    The biases are cast to bfloat16 [P2 Implementation breakdown item 2, Risks item 2]; reading: the
    cast rounds to nearest even, as a float-to-bfloat16 conversion does.  Keeping the top 16 bits
    drops a 16-bit remainder r; the kept part is incremented when r > 0x8000, or r == 0x8000 and the
    kept part is odd.
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    hi = u >> np.uint64(16)
    r = u & np.uint64(0xFFFF)
    up = (r > 0x8000) | ((r == 0x8000) & ((hi & np.uint64(1)) == 1))
    return (hi + up.astype(np.uint64)).astype(np.uint16)


def bias_to_bf16_bits(b, is_fp32):
    """Bias array -> bf16 bit patterns: fp32 input is rounded (f32_to_bf16_bits); bf16 input
    (given as uint16 patterns) passes through unchanged."""
    if is_fp32:
        return f32_to_bf16_bits(b)
    return np.asarray(b, dtype=np.uint16).copy()


def tile_expert_scales(s):
    """Per-expert tiled scales: [E, R, SK] -> [E, mTiles, kTiles, 32, 4, 4].

    Reading: the pages show the tiled layout of one 2-D matrix only; a 3-D expert tensor is tiled one
    expert at a time.  [P3 Key source snippets, untile_cutlass_scale]
    """
    s = np.asarray(s, dtype=np.uint8)
    return np.stack([tile_scales(s[e]) for e in range(s.shape[0])])
