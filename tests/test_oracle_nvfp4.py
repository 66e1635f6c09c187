"""Pins of the oracle's NVFP4 quantizer (the non-E8M0 branch of the pages' converter, with the fix that
elements use the dequantized stored scale): exact cases against a brute-force search, general blocks
against exact rational arithmetic, the effect of the fix, zero blocks and scale saturation.

Page tags as in the oracle: [P3] prhub summary of vLLM PR #43557 (Key source snippets: the NVFP4 branch
of the converter; Review highlights item 2: the dequantized-scale fix).
"""

from fractions import Fraction

import numpy as np
import torch

from oracle import quant as Q
from tests.test_oracle_actquant import brute_e4m3
from tests.test_oracle_quant import brute_nearest_code


def bf16(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_exact_power_of_two_blocks_against_brute_force():
    """Block maximum 6 * 2**j and a power-of-two global scale: vecMax / 6 rounds to exactly 2**j, the
    scale is exact in E4M3, and every element decision is exact -- the nearest E2M1 magnitude of
    |x| / 2**j * 2**-g... computed here by brute force."""
    g = np.random.default_rng(21)
    for gexp in (0, 3, -2):
        gs = 2.0 ** gexp
        n = 400
        j = g.integers(-4, 4, size=n)
        v = g.uniform(-1, 1, size=(n, 16)) * (6.0 * 2.0 ** j)[:, None]
        v[:, 0] = 6.0 * 2.0 ** j
        x = bf16(v)
        q, sc = Q.nvfp4_quantize_ref(x, gs)
        sf = 2.0 ** j * gs
        np.testing.assert_array_equal(Q.E4M3_MAGNITUDES[sc[:, 0]], sf)
        xv = Q.bf16_to_f64(x)
        want = brute_nearest_code((np.abs(xv) * gs / sf[:, None]).reshape(-1)).reshape(n, 16)
        want |= ((x >> 15).astype(np.uint8) << 3)
        np.testing.assert_array_equal(Q.unpack_codes(q), want)
        assert np.all(Q.unpack_codes(q)[:, 0] == 7)  # the maximum lands on 6


def nearest_even(x, table):
    """Exact nearest of a sorted table (Fractions), ties to the even index, beyond the end -> the end."""
    best = 0
    for i, t in enumerate(table):
        d, db = abs(x - t), abs(x - table[best])
        if d < db or (d == db and i % 2 == 0 and best % 2 == 1):
            best = i
    return best


def test_general_blocks_against_exact_arithmetic():
    """Random blocks and global scale: the scale byte is the nearest E4M3 of the exact gs * vecMax / 6,
    and each element code the nearest E2M1 of the exact |x| * gs / SF_deq, except where the exact value
    lies within binary32 rounding (2**-21 relative) of a midpoint."""
    g = np.random.default_rng(5)
    x = bf16(g.standard_t(3, size=(300, 64)) * np.exp2(g.uniform(-6, 6, size=(300, 1))))
    gs = float(np.float32(448 * 6 / float(np.abs(Q.bf16_to_f64(x)).max())))
    q, sc = Q.nvfp4_quantize_ref(x, gs)
    codes = Q.unpack_codes(q) & 7
    e4 = [Fraction(float(m)) for m in Q.E4M3_MAGNITUDES]
    e2 = [Fraction(float(m)) for m in Q.E2M1_MAGNITUDES]
    mid4 = [(a + b) / 2 for a, b in zip(e4, e4[1:])]
    mid2 = [(a + b) / 2 for a, b in zip(e2, e2[1:])]
    near = lambda v, mids: any(abs(v - m) <= m * Fraction(1, 2 ** 21) for m in mids)
    xv = Q.bf16_to_f64(x)
    skipped = total = 0
    G = Fraction(gs)
    for r in range(0, 300, 3):
        for b in range(4):
            blk = xv[r, 16 * b:16 * b + 16]
            sfx = G * Fraction(float(np.abs(blk).max())) / 6
            if not near(sfx, mid4):
                assert sc[r, b] == nearest_even(sfx, e4)
            sfd = e4[sc[r, b]]
            for i in range(16):
                total += 1
                ve = abs(Fraction(float(blk[i]))) * G / sfd if sfd else Fraction(0)
                if near(ve, mid2):
                    skipped += 1
                    continue
                assert codes[r, 16 * b + i] == nearest_even(ve, e2)
    assert skipped < 0.01 * total  # the exemption is rare


def test_elements_use_the_stored_scale():
    """With the fix, reconstruction from the stored scale byte keeps every element within half an E2M1
    step (1/4, 1/2 or 1 times SF_deq / gs, by binade); with the undequantized SF the codes would be
    chosen for another scale, and reconstruction from the stored byte breaks that bound."""
    g = np.random.default_rng(8)
    x = bf16(g.standard_normal((2000, 16)) * np.exp2(g.uniform(-3, 3, size=(2000, 1))))
    gs = 1.0
    q, sc = Q.nvfp4_quantize_ref(x, gs)
    xv = Q.bf16_to_f64(x)
    xh = Q.nvfp4_dequant_ref(q, sc, gs)
    unit = np.repeat(Q.E4M3_MAGNITUDES[sc], 16, axis=-1) / gs
    v = np.abs(xv) / unit
    bound = np.where(v < 2, 0.25, np.where(v <= 4, 0.5, 1.0)) * unit
    assert np.all(np.abs(xh - xv) <= bound * (1 + 2.0 ** -20))
    # the same element rule with the undequantized scale (the behaviour before the fix)
    vm = np.abs(xv).reshape(-1, 16).max(axis=1)
    sf_raw = (np.float32(gs) * (vm.astype(np.float32) * Q.RCP6_F32).astype(np.float32)).astype(np.float64)
    c_raw = Q.e2m1_magnitude_code(np.abs(xv) * gs / np.repeat(sf_raw, 16)[..., None].reshape(xv.shape))
    xh_raw = np.sign(xv) * Q.E2M1_MAGNITUDES[c_raw] * unit
    assert np.any(np.abs(xh_raw - xv) > bound * (1 + 2.0 ** -20))


def test_zero_block_tiny_block_and_scale_saturation():
    x = np.zeros((3, 16), np.uint16)
    x[0, 3] = 0x8000                    # -0.0: magnitude code 0, sign kept
    x[1, :] = bf16(np.full(16, 1e-30))  # scale underflows E4M3 -> 0 -> every code 0
    x[2, :] = bf16(np.linspace(-3000, 3000, 16))
    q, sc = Q.nvfp4_quantize_ref(x, 1.0)
    c = Q.unpack_codes(q)
    assert sc[0, 0] == 0 and np.all(c[0] & 7 == 0) and c[0, 3] == 8
    assert sc[1, 0] == 0 and np.all(c[1] == 0)
    assert sc[2, 0] == 126               # 3000 / 6 = 500 > 448: saturates at 448
    # the E4M3 scale byte agrees with the brute-force search on the binary32 SF
    v = Q.bf16_to_f64(x[2]).astype(np.float32)
    sf = np.float32(np.float32(np.abs(v).max()) * Q.RCP6_F32)
    assert brute_e4m3(np.array([float(sf)]))[0] == 126


def test_tiled_layout_of_nvfp4_scales():
    flat = np.arange(130 * 12, dtype=np.uint32).astype(np.uint8).reshape(130, 12)
    t = Q.nv_tile_scales(flat)
    assert t.shape == (2, 3, 32, 4, 4)
    np.testing.assert_array_equal(Q.untile_scales(t, 130, 12 * 32), flat)
