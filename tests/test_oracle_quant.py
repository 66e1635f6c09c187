"""Pins of the quantization oracle against hand values, closed forms, brute force and invariants.

Page tags as in the oracle: [P3] is the prhub summary of vLLM PR #43557 (E8M0 scale fix).
"""

import math
import struct

import numpy as np
import pytest

from oracle import quant as Q
from tests.exhaustive import exhaustive_blocks, amax_for_scale

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def f32(v):
    return np.float32(v)


def bf16_round(v):
    """Nearest bf16 value of a Python float (via struct, for hand-value tables)."""
    u = struct.unpack("<I", struct.pack("<f", v))[0]
    hi, r = u >> 16, u & 0xFFFF
    if r > 0x8000 or (r == 0x8000 and hi & 1):
        hi += 1
    return struct.unpack("<f", struct.pack("<I", hi << 16))[0]


# ---------------------------------------------------------------- E8M0 scale rule

# The page's missing old-vs-new table spans block maxima 1.2 .. 5.5 [P3 Motivation].  Hand values:
# a maximum m in [1, 1.75) has biased exponent 127 that the 2**21 carry leaves alone, so e = 125;
# in [1.75, 2) the carry lifts it to 128 (e = 126), as does [2, 3.5); [3.5, 7) gives e = 127.
SWEEP = [(1.2, 125), (1.5, 125), (1.6, 125), (1.7, 125), (1.75, 126), (2.0, 126), (2.5, 126),
         (3.0, 126), (3.25, 126), (3.5, 127), (4.0, 127), (4.5, 127), (5.0, 127), (5.5, 127)]


@pytest.mark.parametrize("v,e", SWEEP)
def test_e8m0_sweep_hand_values(v, e):
    assert Q.e8m0_from_amax(f32(v)) == e
    assert Q.e8m0_from_amax(f32(bf16_round(v))) == e
    # ratio max/scale of the new rule stays in [3.5, 7)
    r = v / 2.0 ** (e - 127)
    assert 3.5 <= r < 7


EDGES = [
    (0.0, 0), (-1.0, 0), (2.0 ** -126, 0), (2.0 ** -125, 0), (1.75 * 2.0 ** -125, 1), (2.0 ** -124, 1),
    (0.02, 119), (0.06, 121), (1.0, 125), (6.0, 127), (7.0, 128),
    (bf16_round(3.3895313892515355e38), 253), (float(np.finfo(np.float32).max), 253),
    (2.0 ** -149, 0), (0.75 * 2.0 ** -126, 0),
]


@pytest.mark.parametrize("v,e", EDGES)
def test_e8m0_edge_values(v, e):
    assert Q.e8m0_from_amax(f32(v)) == e


def closed_form_e8m0(a):
    """e = floor(log2 a) + 125 + [significand >= 1.75], clamped to [0, 254], via math.frexp."""
    if a <= 0:
        return 0
    m, ex = math.frexp(a)  # a = m * 2**ex, m in [0.5, 1)
    sig = 2 * m
    e = (ex - 1) + 125 + (1 if sig >= 1.75 else 0)
    return min(max(e, 0), 254)


def test_e8m0_closed_form_random():
    g = np.random.default_rng(7)
    bits = g.integers(1, 0x7F800000, size=200_000, dtype=np.uint64).astype(np.uint32)
    a = bits.view(np.float32)
    got = Q.e8m0_from_amax(a)
    want = np.array([closed_form_e8m0(float(v)) for v in a], dtype=np.uint8)
    np.testing.assert_array_equal(got, want)


def old_rule(a):
    """The superseded rule [P3 Motivation]: biased exponent of max/6 (float64 division; random
    binary32 maxima never land within rounding distance of a binade edge)."""
    m, ex = math.frexp(a / 6.0)
    return ex - 1 + 127


def test_old_rule_is_one_smaller_except_saturating_range():
    """[P3 Motivation]: the old scale is one too small for most inputs, so max/scale lands well above
    6.  Closed form: old = floor(log2 m) + 124 + [sig >= 1.5], new = floor(log2 m) + 125 +
    [sig >= 1.75]; they agree exactly when the significand is in [1.5, 1.75)."""
    g = np.random.default_rng(11)
    a = np.exp2(g.uniform(-60, 60, size=20_000)).astype(np.float32)
    for v in a:
        v = float(v)
        new = int(Q.e8m0_from_amax(f32(v)))
        old = old_rule(v)
        sig = 2 * math.frexp(v)[0]
        assert new - old == (0 if 1.5 <= sig < 1.75 else 1)
        r_old = v / 2.0 ** (old - 127)
        assert 6 <= r_old < 12
    # the sweep rows of the page's table, old rule
    olds = {1.2: 124, 1.5: 125, 1.6: 125, 1.7: 125, 1.75: 125, 2.0: 125, 2.5: 125, 3.0: 126,
            3.25: 126, 3.5: 126, 4.0: 126, 4.5: 126, 5.0: 126, 5.5: 126}
    for v, e in olds.items():
        assert old_rule(v) == e


# ---------------------------------------------------------------- E2M1 element encoding

def brute_nearest_code(v):
    """Nearest of the 8 magnitudes by distance; on an exact tie the even code; beyond 6 -> 6."""
    d = np.abs(v[:, None] - Q.E2M1_MAGNITUDES[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    codes = np.arange(8)[None, :]
    # among tied candidates prefer the even code
    score = np.where(cand, np.where(codes % 2 == 0, 0, 1), 9)
    return np.argmin(score * 8 + codes, axis=1).astype(np.uint8)


def test_e2m1_midpoints():
    v = np.array([0.0, 0.25, 0.2500001, 0.75, 0.7499999, 1.25, 1.2500001, 1.75, 2.5, 2.5000001,
                  3.5, 3.4999999, 5.0, 5.0000001, 6.0, 6.9, 100.0])
    want = np.array([0, 0, 1, 2, 1, 2, 3, 4, 4, 5, 6, 5, 6, 7, 7, 7, 7])
    np.testing.assert_array_equal(Q.e2m1_magnitude_code(v), want)
    np.testing.assert_array_equal(brute_nearest_code(v), want)


@pytest.mark.parametrize("chunk", range(8))
def test_quantize_elements_exhaustive(chunk):
    """Every finite bf16 pattern under every scale exponent it can meet, against the brute-force
    nearest-magnitude search."""
    for e in range(chunk, 254, 8):
        x = exhaustive_blocks(e)
        q, s = Q.quantize_ref(x)
        assert np.all(s[:, 0] == e)
        codes = Q.unpack_codes(q)
        v = Q.bf16_to_f64(x & 0x7FFF) * 2.0 ** (127 - e)
        want = brute_nearest_code(v.reshape(-1)).reshape(x.shape)
        want |= ((x >> 15).astype(np.uint8) << 3)
        np.testing.assert_array_equal(codes, want, err_msg=f"e={e}")


def test_amax_for_scale_is_largest():
    for e in range(254):
        top = amax_for_scale(e)
        assert Q.e8m0_from_amax(Q.bf16_to_f64(np.array([top], np.uint16)).astype(np.float32))[0] == e
        if e < 253:
            nxt = np.array([top + 1], np.uint16)
            assert Q.e8m0_from_amax(Q.bf16_to_f64(nxt).astype(np.float32))[0] == e + 1


def test_nibble_packing_order():
    """Reading fixed by this library's ABI (pages silent): element 2j -> low nibble, 2j+1 -> high."""
    x = np.zeros((1, 32), np.uint16)
    x[0, 0] = 0x3F80  # 1.0 -> amax 1.0 -> e = 125 -> v = 4 -> code 6
    x[0, 1] = 0xBF00  # -0.5 -> v = 2 -> code 4 | 8
    q, s = Q.quantize_ref(x)
    assert s[0, 0] == 125
    assert q[0, 0] == (6 | (0xC << 4))
    # sign kept on a code of magnitude 0
    x[0, 2] = 0x8000
    q, _ = Q.quantize_ref(x)
    assert q[0, 1] & 0xF == 0x8


# ---------------------------------------------------------------- invariants

def _student_blocks(n, seed):
    g = np.random.default_rng(seed)
    v = g.standard_t(3, size=(n, 32)) * np.exp2(g.uniform(-20, 20, size=(n, 1)))
    import torch
    return torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_invariants_ratio_saturation_error():
    x = _student_blocks(40_000, 3)
    q, s = Q.quantize_ref(x)
    xv = Q.bf16_to_f64(x)
    amax = np.abs(xv).max(axis=1)
    scale = np.ldexp(1.0, s[:, 0].astype(int) - 127)
    ok = s[:, 0] >= 1
    r = amax[ok] / scale[ok]
    assert r.min() >= 3.5 and r.max() < 7  # max is 6.96875 for bf16
    # a block saturates (its max lands above 6) iff the max's significand is in (1.5, 1.75)
    sig = amax / np.exp2(np.floor(np.log2(np.where(amax > 0, amax, 1))))
    sat = (amax / scale) > 6
    np.testing.assert_array_equal(sat[ok], ((sig > 1.5) & (sig < 1.75))[ok])
    # reconstruction error bound per element, in units of the block scale
    xh = Q.dequant_ref(q, s)
    v = np.abs(xv) / scale[:, None]
    err = np.abs(xh - xv) / scale[:, None]
    bound = np.where(v < 2, 0.25, np.where(v <= 4, 0.5, 1.0))
    assert np.all(err <= bound + 1e-12)


def test_idempotence():
    x = _student_blocks(20_000, 5)
    q, s = Q.quantize_ref(x)
    xh = Q.dequant_ref(q, s)
    # dequantized values have one mantissa bit, exact in bf16 for these ranges
    xb = (xh.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(Q.bf16_to_f64(xb), xh)
    q2, s2 = Q.quantize_ref(xb)
    np.testing.assert_array_equal(s2, s)
    np.testing.assert_array_equal(q2, q)


def test_no_whole_block_saturation_on_extreme_inputs():
    """Extreme magnitudes never saturate a whole block [P3 Implementation breakdown, item 3].  Exact
    form: every element of a block saturates only when all of them lie in (5, 7) * scale."""
    g = np.random.default_rng(9)
    for lo, hi in [(-120, -100), (100, 120), (-126, 127)]:
        v = g.standard_normal((5000, 32)) * np.exp2(g.uniform(lo, hi, size=(5000, 1)))
        import torch
        x = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        q, s = Q.quantize_ref(x)
        codes = Q.unpack_codes(q) & 7
        assert not np.any(np.all(codes == 7, axis=1))
    # a constant block whose value has significand in (1.5, 1.75) is the case that does saturate
    x = np.full((1, 32), 0x3FCD, np.uint16)  # 1.6015625
    q, s = Q.quantize_ref(x)
    assert np.all(Q.unpack_codes(q) == 7)


def test_zero_block_and_tiny_scale_reading():
    x = np.zeros((2, 32), np.uint16)
    x[1, 5] = 0x0001  # smallest bf16 subnormal: e = 0, v = 2**-133 * 2**127 -> code 0
    x[1, 6] = 0x0050  # 80 * 2**-133 = 1.25 * 2**-127 -> v = 1.25 -> code 2 (tie to even)
    q, s = Q.quantize_ref(x)
    assert s[0, 0] == 0 and np.all(q[0] == 0)
    c = Q.unpack_codes(q[1:])[0]
    assert s[1, 0] == 0 and c[5] == 0 and c[6] == 2
    # reading: dequant uses 2**(e - 127) also for e = 0
    assert Q.dequant_ref(q[1:], s[1:])[0, 6] == 1.0 * 2.0 ** -127


def test_dequant_code_table():
    s = np.array([[127]], np.uint8)
    q = np.zeros((1, 16), np.uint8)
    q[0, :8] = np.arange(16, dtype=np.uint8)[0::2] | (np.arange(16, dtype=np.uint8)[1::2] << 4)
    vals = Q.dequant_ref(q, s)[0, :16]
    want = [0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6]
    np.testing.assert_array_equal(vals, want)


# ---------------------------------------------------------------- tiled scales

def test_tiled_offset_hand_example():
    """M = K = 256: K/32 = 8 scale columns, 2 k-tiles.  flat[37, 5]: mT 0, iM 1, oM 5, kT 1, iK 1 ->
    byte ((0*2 + 1)*32 + 5)*16 + 1*4 + 1 = 597."""
    flat = np.zeros((256, 8), np.uint8)
    flat[37, 5] = 0xAB
    t = Q.tile_scales(flat).reshape(-1)
    assert t.size == 2 * 2 * 512
    assert np.nonzero(t)[0].tolist() == [597]
    assert t[597] == 0xAB


@pytest.mark.parametrize("M,SK", [(1, 1), (127, 3), (128, 4), (129, 5), (300, 8), (256, 224), (64, 56)])
def test_tile_untile_round_trip(M, SK):
    g = np.random.default_rng(M * 1000 + SK)
    flat = g.integers(1, 256, size=(M, SK), dtype=np.uint8)
    t = Q.tile_scales(flat)
    assert t.shape == Q.tiled_scale_shape(M, SK * 32)
    np.testing.assert_array_equal(Q.untile_scales(t, M, SK * 32), flat)
    # padding bytes are zero and every real byte appears once
    assert np.count_nonzero(t) == M * SK
