"""Pins of the oracle's activation quantizers (the MoE layer's quantized-activation variants) and of
the tiled-scale untile, against the pages' own recipe, closed forms and brute force.

Page tags as in the oracle: [P2] prhub report of vLLM PR #51038 (the FlashInfer CUTLASS MXFP4 conversion
with its MXFP8-activation variant); [P3] prhub summary of vLLM PR #43557 (E8M0 scale fix; the untile
helper; the experts-quant tests).
"""

import math

import numpy as np
import pytest
import torch

from oracle import quant as Q
from tests.test_oracle_quant import brute_nearest_code


# ---------------------------------------------------------------- untile, the page's recipe

def page_untile(raw, rows, K):
    """The page's untile helper restated: view the first padded_M * padded_SK bytes as
    [mTiles, kTiles, 32, 4, 4], permute axes (0, 3, 2, 1, 4), reshape to (padded_M, padded_SK) and crop
    to (rows, K / 32).  [P3 Key source snippets, untile_cutlass_scale]"""
    sk = K // 32
    mt, kt = (rows + 127) // 128, (sk + 3) // 4
    t = np.asarray(raw, np.uint8).reshape(-1)[: mt * 128 * kt * 4].reshape(mt, kt, 32, 4, 4)
    return np.ascontiguousarray(t.transpose(0, 3, 2, 1, 4)).reshape(mt * 128, kt * 4)[:rows, :sk]


@pytest.mark.parametrize("rows,SK", [(1, 1), (127, 3), (128, 4), (129, 5), (300, 8), (256, 224)])
def test_untile_equals_the_pages_permutation(rows, SK):
    g = np.random.default_rng(rows + 7 * SK)
    raw = g.integers(0, 256, size=int(np.prod(Q.tiled_scale_shape(rows, SK * 32))), dtype=np.uint8)
    np.testing.assert_array_equal(Q.untile_scales(raw, rows, SK * 32), page_untile(raw, rows, SK * 32))
    flat = g.integers(0, 256, size=(rows, SK), dtype=np.uint8)
    np.testing.assert_array_equal(page_untile(Q.tile_scales(flat), rows, SK * 32), flat)


# ---------------------------------------------------------------- MXFP4 of binary32 values

def test_values_quantizer_equals_bf16_quantizer_on_bf16_inputs():
    """On bf16-representable inputs the binary32 quantizer is the (exhaustively pinned) bf16 one."""
    g = np.random.default_rng(3)
    v = g.standard_t(3, size=(3000, 64)) * np.exp2(g.uniform(-30, 30, size=(3000, 1)))
    bits = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    q, s = Q.quantize_ref(bits)
    codes, s2 = Q.quantize_values_ref(Q.bf16_to_f64(bits).astype(np.float32))
    np.testing.assert_array_equal(s2, s)
    np.testing.assert_array_equal(codes, Q.unpack_codes(q))


def test_values_quantizer_brute_force_on_binary32():
    """Inputs with 24-bit significands (not bf16): every code against a nearest-of-8 search of the
    scaled magnitude, computed per block from math.frexp."""
    g = np.random.default_rng(4)
    x = (g.standard_normal((2000, 32)) * np.exp2(g.uniform(-10, 10, size=(2000, 1)))).astype(np.float32)
    x[0, :] = 0.0
    x[1, 3] = -0.0
    codes, s = Q.quantize_values_ref(x)
    for b in range(x.shape[0]):
        amax = float(np.abs(x[b]).max())
        if amax == 0:
            e = 0
        else:
            m, ex = math.frexp(amax)
            e = min(max((ex - 1) + 125 + (1 if 2 * m >= 1.75 else 0), 0), 254)
        assert s[b, 0] == e
        v = np.abs(x[b].astype(np.float64)) * 2.0 ** (127 - e)
        want = brute_nearest_code(v) | (np.signbit(x[b]).astype(np.uint8) << 3)
        np.testing.assert_array_equal(codes[b], want)
    np.testing.assert_array_equal(Q.dequant_codes_ref(codes[:1], s[:1]), np.zeros((1, 32)))


# ---------------------------------------------------------------- E4M3 elements

def brute_e4m3(v):
    """Nearest of the 127 E4M3 magnitudes by distance, the even code on an exact tie, beyond the
    largest -> the largest."""
    d = np.abs(v[:, None] - Q.E4M3_MAGNITUDES[None, :])
    dmin = d.min(axis=1, keepdims=True)
    codes = np.arange(127)[None, :]
    score = np.where(d == dmin, np.where(codes % 2 == 0, 0, 1), 9)
    return np.argmin(score * 128 + codes, axis=1).astype(np.uint8)


def test_e4m3_table_hand_values():
    M = Q.E4M3_MAGNITUDES
    assert M.size == 127 and M[0] == 0 and M[1] == 2.0 ** -9 and M[7] == 7 * 2.0 ** -9
    assert M[8] == 2.0 ** -6 and M[0x38] == 1.0 and M[0x77] == 240.0 and M[126] == 448.0
    assert np.all(np.diff(M) > 0)  # codes are ordered by value


def test_e4m3_midpoints_and_saturation():
    v = np.array([0.0, 2.0 ** -10, 2.0 ** -10 * 1.0001, 1.5 * 2.0 ** -9, 2.5 * 2.0 ** -9, 1.0625, 1.0625 * 1.0000001,
                  1.1875, 432.0, 440.0, 447.9, 448.0, 464.0, 1000.0])
    want = np.array([0, 0, 1, 2, 2, 0x38, 0x39, 0x3A, 126, 126, 126, 126, 126, 126])
    np.testing.assert_array_equal(Q.e4m3_magnitude_code(v), want)
    np.testing.assert_array_equal(brute_e4m3(v), want)


def test_e4m3_exhaustive_over_bf16_magnitudes():
    """Every non-negative finite bf16 value below 512 (8 significant bits, so every E4M3 midpoint is
    among them) against the brute-force search."""
    bits = np.arange(0, 0x4400, dtype=np.uint16)  # up to 512
    v = Q.bf16_to_f64(bits)
    np.testing.assert_array_equal(Q.e4m3_magnitude_code(v), brute_e4m3(v))


# ---------------------------------------------------------------- E8M0 rule for E4M3 blocks

def closed_form_e8m0_e4m3(a):
    """floor(log2 a) + 127 - 8 + [significand >= 1.75], clamped to [0, 254]."""
    if a <= 0:
        return 0
    m, ex = math.frexp(a)
    return min(max((ex - 1) + 119 + (1 if 2 * m >= 1.75 else 0), 0), 254)


def test_e4m3_scale_rule_closed_form_and_relation_to_the_pages_rule():
    g = np.random.default_rng(8)
    bits = g.integers(1, 0x7F800000, size=100_000, dtype=np.uint64).astype(np.uint32)
    a = bits.view(np.float32)
    e8 = Q.e8m0_for_e4m3(a)
    want = np.array([closed_form_e8m0_e4m3(float(v)) for v in a], dtype=np.uint8)
    np.testing.assert_array_equal(e8, want)
    # the same rounded binade as the pages' MXFP4 rule, six binades lower (2 vs 8 element exponent)
    e4 = Q.e8m0_from_amax(a).astype(int)
    np.testing.assert_array_equal(e8.astype(int), np.maximum(e4 - 6, 0))
    assert Q.e8m0_for_e4m3(np.float32(0.0)) == 0 and Q.e8m0_for_e4m3(np.float32(-3.0)) == 0
    # 447 keeps its binade (ratio 447); 448 = 1.75 * 2**8 rounds up (ratio 224); 1.0 -> 2**-8 scale
    assert Q.e8m0_for_e4m3(np.float32(447.0)) == 127 and Q.e8m0_for_e4m3(np.float32(448.0)) == 128
    assert Q.e8m0_for_e4m3(np.float32(1.0)) == 119


def test_mxfp8_block_invariants():
    """The block maximum maps into [224, 448) (no element saturates); each element's error is at most
    half an E4M3 step of its own binade (or half the subnormal step); quantizing the dequantized values
    again is the identity, except for blocks whose maximum rounded up to 448 = 1.75 * 2**8: that value
    is itself rounded up by the rule, so those blocks come back one binade up (values below the new
    subnormal step may round once more)."""
    g = np.random.default_rng(12)
    x = (g.standard_t(3, size=(20000, 32)) * np.exp2(g.uniform(-40, 40, size=(20000, 1)))).astype(np.float32)
    codes, s = Q.mxfp8_quantize_values_ref(x)
    scale = np.ldexp(1.0, s[:, 0].astype(int) - 127)
    amax = np.abs(x).max(axis=1).astype(np.float64)
    r = amax / scale
    assert r.min() >= 224 and r.max() < 448
    xh = Q.mxfp8_dequant_ref(codes, s)
    v = np.abs(x.astype(np.float64)) / scale[:, None]
    step = np.where(v < 2.0 ** -6, 2.0 ** -9, np.exp2(np.floor(np.log2(np.maximum(v, 2.0 ** -6))) - 3))
    assert np.all(np.abs(xh - x) / scale[:, None] <= step / 2 * (1 + 1e-12))
    c2, s2 = Q.mxfp8_quantize_values_ref(xh.astype(np.float32))
    top = (np.abs(xh) / scale[:, None]).max(axis=1) == 448.0
    assert 0 < np.count_nonzero(top) < top.size
    np.testing.assert_array_equal(s2[~top], s[~top])
    np.testing.assert_array_equal(c2[~top], codes[~top])
    np.testing.assert_array_equal(s2[top].astype(int), s[top].astype(int) + 1)
    # one binade up, the values keep their bits except where the subnormal step doubled
    d2 = np.abs(Q.mxfp8_dequant_ref(c2, s2) - xh)[top]
    sub = 2.0 ** -9 * np.ldexp(1.0, s2[top, :1].astype(int) - 127)
    assert np.all(d2 <= sub / 2) and np.count_nonzero(d2) < 0.01 * d2.size
