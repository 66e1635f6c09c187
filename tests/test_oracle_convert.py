"""Pins of the checkpoint-conversion oracle: the page's worked swap example, involution, textbook
bf16 rounding cases and an independent library cast.

[P2] is the prhub report of vLLM PR #51038 "[Bugfix][Quantization] Fix MXFP4 conversion for
FlashInfer CUTLASS".
"""

import os

import numpy as np
import pytest
import torch

from oracle import convert as C
from oracle import quant as Q

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "swap_probe.txt")


def load_swap_probe():
    ins, outs = {}, {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        head, shape, vals = [p.strip() for p in line.split("|")]
        kind, name = head.split()
        arr = np.array([int(v) for v in vals.split()]).reshape([int(s) for s in shape.split(",")])
        (ins if kind == "in" else outs)[name] = arr
    return ins, outs


def test_swap_probe_matches_page_example():
    ins, outs = load_swap_probe()
    np.testing.assert_array_equal(C.swap_w13_w31(ins["w13"].astype(np.uint8)), outs["w13"])
    np.testing.assert_array_equal(C.swap_w13_w31(ins["w13_scale"].astype(np.uint8)), outs["w13_scale"])
    b13 = C.bias_to_bf16_bits(C.swap_b13_b31(ins["w13_bias"].astype(np.float32)), is_fp32=True)
    np.testing.assert_array_equal(Q.bf16_to_f64(b13), outs["w13_bias"])
    b2 = C.bias_to_bf16_bits(ins["w2_bias"].astype(np.float32), is_fp32=True)
    np.testing.assert_array_equal(Q.bf16_to_f64(b2), outs["w2_bias"])
    # w2 and its scale are not touched by the conversion
    np.testing.assert_array_equal(ins["w2"], outs["w2"])
    np.testing.assert_array_equal(ins["w2_scale"], outs["w2_scale"])


def test_swap_is_an_involution_and_moves_halves():
    g = np.random.default_rng(1)
    w = g.integers(0, 256, size=(3, 10, 6), dtype=np.uint8)
    s = C.swap_w13_w31(w)
    np.testing.assert_array_equal(C.swap_w13_w31(s), w)
    np.testing.assert_array_equal(s[:, :5], w[:, 5:])
    np.testing.assert_array_equal(s[:, 5:], w[:, :5])
    b = g.standard_normal((3, 10)).astype(np.float32)
    np.testing.assert_array_equal(C.swap_b13_b31(C.swap_b13_b31(b)), b)
    with pytest.raises(ValueError):
        C.swap_w13_w31(np.zeros((1, 3, 2), np.uint8))


def test_bf16_rounding_textbook_cases():
    # 1 + 2**-8 is half an ulp above 1.0: tie, kept part even -> 1.0
    # 1 + 3 * 2**-8 is half an ulp above 1 + 2**-7 (odd): tie -> 1 + 2**-6
    # 1 + 2**-8 + 2**-20 is above the tie -> 1 + 2**-7
    cases = [(1 + 2 ** -8, 1.0), (1 + 3 * 2 ** -8, 1 + 2 ** -6), (1 + 2 ** -8 + 2 ** -20, 1 + 2 ** -7),
             (-(1 + 2 ** -8), -1.0), (0.0, 0.0), (2.0 ** -130, 2.0 ** -130), (3.0, 3.0)]
    for v, want in cases:
        got = Q.bf16_to_f64(C.f32_to_bf16_bits(np.array([v], np.float32)))[0]
        assert got == want, (v, got, want)


def test_bf16_rounding_matches_torch_cast():
    g = np.random.default_rng(2)
    bits = g.integers(0, 0x7F7F0000, size=300_000, dtype=np.uint64).astype(np.uint32)
    bits[::2] |= 0x80000000
    x = bits.view(np.float32)
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(C.f32_to_bf16_bits(x), want)


def test_expert_tiling_equals_stacked_tiling_when_rows_fill_tiles():
    """Reading: 3-D scales are tiled per expert; with rows a multiple of 128 that is the same as
    tiling the stacked [E * rows, SK] matrix."""
    g = np.random.default_rng(3)
    s = g.integers(0, 256, size=(3, 256, 8), dtype=np.uint8)
    per = C.tile_expert_scales(s).reshape(-1)
    stacked = Q.tile_scales(s.reshape(-1, 8)).reshape(-1)
    np.testing.assert_array_equal(per, stacked)
