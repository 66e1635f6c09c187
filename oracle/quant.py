"""Oracle: OCP-MX MXFP4 block quantization, dequantization and the tiled scale layout.

Test infrastructure only (see the package docstring).  Pure NumPy; exact arithmetic:
bf16 inputs are widened exactly, the scaled magnitude |x| * 2**(127 - e) is an exact float64 product,
and every rounding decision is a comparison against exact midpoints.
"""

import numpy as np

BLOCK = 32
"""Elements per scale block along K.  [P3 Key source snippets, test_mxfp4_moe.py: the untile helper
divides K by the MXFP4 block size of 32]  [DEF: 32-element blocks]"""

E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
"""Magnitude of each 3-bit E2M1 code (OCP-MX FP4: 1 sign, 2 exponent, 1 mantissa bit, bias 1).
The largest magnitude 6.0 is the one [P3 Motivation] compares max/scale against."""


def bf16_to_f64(bits):
    """Exact value of bf16 bit patterns (uint16) as float64: the pattern is the top half of a binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e8m0_from_amax(amax):
    """E8M0 scale byte for blocks whose largest magnitude is ``amax`` (binary32 values).

    [P3 Implementation breakdown, item 1; Key source snippets: the reference helper in the MoE test
    and the UE8M0_SF branch of the FP16/BF16 -> FP4 converter state the same rule]:
      * a block maximum that is not positive gives 0;
      * otherwise add 2**21 to the binary32 bit pattern of the maximum (a significand of 1.75 or more
        then carries into the next binade) and read the biased exponent B of the sum;
      * the scale exponent is B - 2, floored at 0 and capped at 254.
    For a positive finite maximum the pattern is below 0x7F800000, so the sum stays below 2**31 and
    B is simply the sum shifted right by 23.
    """
    a = np.asarray(amax, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.int64)
    biased = (bits + (1 << 21)) >> 23
    e = np.minimum(np.maximum(biased - 2, 0), 254)
    return np.where(a > 0, e, 0).astype(np.uint8)


def e2m1_magnitude_code(v):
    """E2M1 magnitude code of v >= 0 (float64), round to nearest, ties to the even code, saturating.

    [DEF: E2M1 elements, round-to-nearest-even, saturating at +-6]  The representable magnitudes are
    E2M1_MAGNITUDES; the midpoints between neighbours are 0.25, 0.75, 1.25, 1.75, 2.5, 3.5 and 5.
    On a midpoint the neighbour with the even code wins (0.25 -> 0, 0.75 -> 1.0, 1.25 -> 1.0,
    1.75 -> 2.0, 2.5 -> 2.0, 3.5 -> 4.0, 5 -> 4.0), and anything above 5 becomes 6.0 (code 7).
    """
    v = np.asarray(v, dtype=np.float64)
    c = (v > 0.25).astype(np.uint8)
    c += v >= 0.75
    c += v > 1.25
    c += v >= 1.75
    c += v > 2.5
    c += v >= 3.5
    c += v > 5.0
    return c


def quantize_ref(x_bits):
    """MXFP4 quantization of a bf16 matrix.

    x_bits: uint16 [M, K] bf16 bit patterns, K a multiple of 32.
    Returns (q, scales): q uint8 [M, K/2] packed E2M1 codes, scales uint8 [M, K/32] E8M0 bytes.

    Steps for every 32-element block along K:
      1. amax = max |x| over the block (the pages reduce the block with a max over the lanes' values;
         reading: the maximum of magnitudes, as the not-positive branch of the reference implies)
         [P3 Key source snippets].
      2. e = e8m0_from_amax(amax).
      3. v = |x| * 2**(127 - e), exact in float64; magnitude code by e2m1_magnitude_code [DEF].
      4. sign bit 0x8 set when the input's sign bit is set, also when the magnitude code is 0
         (reading: the sign is kept; the pages are silent).
      5. two codes per byte, element 2j in the low nibble and 2j+1 in the high nibble
         (reading: the pages only say "packed 4-bit" [P1 Implementation breakdown] and keep K/2 as the
         last dimension [P2 Key source snippets, the conversion test's w13 of shape [1, 4, 4]]).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    M, K = x_bits.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    blocks = x_bits.reshape(M, K // BLOCK, BLOCK)
    mag = bf16_to_f64(blocks & np.uint16(0x7FFF))
    amax = mag.max(axis=-1)  # a bf16 value, so its binary32 form is exact
    e = e8m0_from_amax(amax.astype(np.float32))
    v = mag * np.ldexp(1.0, 127 - e.astype(np.int64))[..., None]
    code = e2m1_magnitude_code(v)
    code |= ((blocks >> np.uint16(15)).astype(np.uint8) << np.uint8(3))
    code = code.reshape(M, K)
    q = (code[:, 0::2] | (code[:, 1::2] << np.uint8(4))).astype(np.uint8)
    return q, e


def unpack_codes(q):
    """Inverse of the nibble packing of quantize_ref: uint8 [..., K/2] -> uint8 codes [..., K]."""
    q = np.asarray(q, dtype=np.uint8)
    out = np.empty(q.shape[:-1] + (q.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = q & np.uint8(0xF)
    out[..., 1::2] = q >> np.uint8(4)
    return out


def dequant_ref(q, scales):
    """x_hat = (-1)**s * E2M1_MAGNITUDES[code & 7] * 2**(e - 127), float64.

    [P3 Key source snippets: the kernel rebuilds the scale from the E8M0 byte as 2**(e - 127); the
    pages' test checks the reconstruction error]  Reading: 2**(e - 127) for every e including 0
    (the kernel snippet's bit-shift rebuild would give +0.0 for e = 0; the two differ only for blocks
    whose maximum is below about 2**-124).
    q: uint8 [..., K/2], scales: uint8 [..., K/32].
    """
    codes = unpack_codes(q)
    mag = E2M1_MAGNITUDES[codes & 7]
    sign = np.where(codes & 8, -1.0, 1.0)
    s = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127)
    s = np.repeat(s, BLOCK, axis=-1)
    return sign * mag * s


def tiled_scale_shape(M, K):
    """[mTiles, kTiles, 32, 4, 4] for an [M, K] matrix: 128 rows by 4 scale columns per 512-byte tile.
    [P3 Key source snippets, untile_cutlass_scale]"""
    sk = K // BLOCK
    return ((M + 127) // 128, (sk + 3) // 4, 32, 4, 4)


def tile_scales(flat):
    """Flat E8M0 scales [M, SK] -> tiled uint8 [mTiles, kTiles, 32, 4, 4].

    The byte at tiled[mT, kT, oM, iM, iK] is flat[mT*128 + iM*32 + oM, kT*4 + iK]; padding rows
    (>= M) and padding columns (>= SK) hold 0 (reading: the pages only read the first
    padded_M*padded_SK bytes back).  This is the layout whose inverse the pages give as a permute of
    axes (0, 3, 2, 1, 4) followed by a reshape to (padded_M, padded_SK).  [P3 Key source snippets,
    untile_cutlass_scale]
    """
    flat = np.asarray(flat, dtype=np.uint8)
    M, SK = flat.shape
    mt, kt = (M + 127) // 128, (SK + 3) // 4
    out = np.zeros((mt, kt, 32, 4, 4), dtype=np.uint8)
    r, c = np.indices((M, SK))
    out[r // 128, c // 4, r % 32, (r % 128) // 32, c % 4] = flat
    return out


def tiled_offset(r, c, K):
    """Byte offset of flat scale [r, c] in the tiled layout of a matrix with K columns:
    ((mT * kTiles + kT) * 32 + oM) * 16 + iM * 4 + iK with mT = r // 128, iM = (r % 128) // 32,
    oM = r % 32, kT = c // 4, iK = c % 4.  [P3 Key source snippets, untile_cutlass_scale: the tiles are
    [numMTiles, numKTiles, 32 (outer M), 4 (inner M), 4 (inner K)]; reading 9 of the labels]"""
    kt = (K // BLOCK + 3) // 4
    r, c = np.asarray(r), np.asarray(c)
    return (((r // 128) * kt + c // 4) * 32 + r % 32) * 16 + ((r % 128) // 32) * 4 + c % 4


def untile_scales(tiled, rows, K):
    """Tiled scale bytes -> flat [rows, K/32]: element [r, c] is the byte at tiled_offset(r, c, K);
    padding bytes are ignored.  The inverse of tile_scales.  [P3 Key source snippets,
    untile_cutlass_scale]"""
    b = np.asarray(tiled, dtype=np.uint8).reshape(-1)
    r, c = np.indices((rows, K // BLOCK))
    return b[tiled_offset(r, c, K)]


# ------------------------------------------------------------------------------------------------
# Activation quantizers of the MoE layer's quantized-activation variants.

def quantize_values_ref(values):
    """MXFP4 quantization of binary32 values [M, K] (K a multiple of 32), the element rule and the
    E8M0 rule of quantize_ref applied to binary32 inputs: amax is the largest binary32 magnitude of
    the block (exact), e = e8m0_from_amax(amax), v = |x| * 2**(127 - e) exact in float64, code by
    e2m1_magnitude_code, sign bit 0x8 from the value's sign bit.  Returns (codes uint8 [M, K] unpacked,
    scales uint8 [M, K/32]).  [P3 Implementation breakdown item 3: the experts-quant kernel quantizes
    MoE activations with the same E8M0 rule]"""
    x = np.asarray(values, dtype=np.float32)
    M, K = x.shape
    blocks = x.reshape(M, K // BLOCK, BLOCK)
    mag = np.abs(blocks).astype(np.float64)
    e = e8m0_from_amax(np.abs(blocks).max(axis=-1))
    v = mag * np.ldexp(1.0, 127 - e.astype(np.int64))[..., None]
    code = e2m1_magnitude_code(v) | (np.signbit(blocks).astype(np.uint8) << np.uint8(3))
    return code.reshape(M, K), e


def dequant_codes_ref(codes, scales):
    """Unpacked E2M1 codes [..., K] and E8M0 scales [..., K/32] -> float64 values (as dequant_ref)."""
    codes = np.asarray(codes, dtype=np.uint8)
    mag = E2M1_MAGNITUDES[codes & 7]
    sign = np.where(codes & 8, -1.0, 1.0)
    s = np.repeat(np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127), BLOCK, axis=-1)
    return sign * mag * s


E4M3_MAGNITUDES = np.array([m / 8 * 2.0 ** -6 for m in range(8)] +
                           [(1 + m / 8) * 2.0 ** (E - 7) for E in range(1, 16) for m in range(8)])[:127]
"""Magnitude of each 7-bit OCP FP8 E4M3 code (4 exponent bits, bias 7, 3 mantissa bits; exponent 0 is
subnormal; no infinities, code 0x7F is NaN and left out): codes 0..126, largest 448 = 1.75 * 2**8."""

_E4M3_MID = (E4M3_MAGNITUDES[1:] + E4M3_MAGNITUDES[:-1]) / 2


def e4m3_magnitude_code(v):
    """E4M3 magnitude code of v >= 0 (float64): the nearest magnitude, the even code on an exact
    midpoint, 448 (code 126) for anything beyond.  [DEF: OCP FP8 E4M3 elements of MXFP8, rounded to
    nearest even]"""
    v = np.asarray(v, dtype=np.float64)
    c = np.searchsorted(_E4M3_MID, v, side="left")  # midpoints strictly below v
    on_mid = (c < _E4M3_MID.size) & (_E4M3_MID[np.minimum(c, _E4M3_MID.size - 1)] == v)
    c = np.where(on_mid & (c % 2 == 1), c + 1, c)
    return c.astype(np.uint8)


def e8m0_for_e4m3(amax):
    """E8M0 scale byte of an MXFP8 (E4M3) block, the pages' rule carried over to E4M3 elements
    (reading; the pages give the rule for E2M1 only): the same round-up of the block maximum at a
    significand of 1.75, minus the largest element exponent, 8 for E4M3 (448 = 1.75 * 2**8) where E2M1
    subtracts 2 (6 = 1.5 * 2**2).  So e = B - 8 with B as in e8m0_from_amax, floored at 0, capped at
    254, and 0 for a maximum that is not positive.  The maximum then maps into [224, 448): E4M3's
    largest magnitude is 1.75 * 2**8, exactly the round-up threshold, so no element saturates."""
    a = np.asarray(amax, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.int64)
    biased = (bits + (1 << 21)) >> 23
    e = np.minimum(np.maximum(biased - 8, 0), 254)
    return np.where(a > 0, e, 0).astype(np.uint8)


def mxfp8_quantize_values_ref(values):
    """MXFP8 quantization of binary32 values [M, K]: per 32-element block e = e8m0_for_e4m3(amax),
    v = |x| * 2**(127 - e) exact in float64, code = e4m3_magnitude_code(v) | sign bit 0x80.
    Returns (codes uint8 [M, K], scales uint8 [M, K/32]).  [P2 Implementation breakdown item 3: the
    MXFP8-activation variant of the FlashInfer CUTLASS MXFP4 MoE backend]"""
    x = np.asarray(values, dtype=np.float32)
    M, K = x.shape
    blocks = x.reshape(M, K // BLOCK, BLOCK)
    e = e8m0_for_e4m3(np.abs(blocks).max(axis=-1))
    v = np.abs(blocks).astype(np.float64) * np.ldexp(1.0, 127 - e.astype(np.int64))[..., None]
    code = e4m3_magnitude_code(v) | (np.signbit(blocks).astype(np.uint8) << np.uint8(7))
    return code.reshape(M, K), e


def mxfp8_dequant_ref(codes, scales):
    """E4M3 codes [..., K] and E8M0 scales [..., K/32] -> float64 values."""
    codes = np.asarray(codes, dtype=np.uint8)
    mag = E4M3_MAGNITUDES[codes & 0x7F]
    sign = np.where(codes & 0x80, -1.0, 1.0)
    s = np.repeat(np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127), BLOCK, axis=-1)
    return sign * mag * s


# ------------------------------------------------------------------------------------------------
# NVFP4: the sibling format the same converter handles when the scale is not E8M0.

NV_BLOCK = 16
"""Elements per NVFP4 scale block (reading: the pages show the NVFP4 branch of the converter but not
its block size; NVFP4 blocks hold 16 elements)."""

RCP6_F32 = np.float32(1.0) / np.float32(6.0)
"""The binary32 reciprocal of 6 the NVFP4 scale multiplies by (reading: the page's reciprocal of 6.0f,
taken as the correctly rounded binary32 value 0x3E2AAAAB)."""


def nvfp4_quantize_ref(x_bits, global_scale):
    """NVFP4 quantization of a bf16 matrix [M, K] (K a multiple of 16) with a binary32 global scale.

    [P3 Implementation breakdown item 1 and Key source snippets, the non-UE8M0 branch of the converter;
    Review highlights item 2, the fix that makes the element scale the dequantized stored scale]
    Per 16-element block, every step in binary32 as the converter computes it:
      1. vecMax = max |x| (exact);
      2. SF = global_scale * (vecMax * RCP6_F32), two binary32 roundings;
      3. the stored scale byte is SF as E4M3, nearest even, saturating at 448 (e4m3_magnitude_code);
      4. SF_deq = that byte's value (the fix: elements use the dequantized scale);
      5. r = global_scale / SF_deq in binary32 (0 when SF_deq is 0; reading, the page does not show the
         element step: elements are divided by SF_deq / global_scale, the scale they dequantize with);
      6. code = E2M1 of |x| * r (binary32 product, then nearest even, saturating at 6), sign bit 0x8 from
         x (also for magnitude 0, reading 3 of the MXFP4 quantizer), two codes per byte as quantize_ref.
    Returns (q uint8 [M, K/2], scale codes uint8 [M, K/16]).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    M, K = x_bits.shape
    if K % NV_BLOCK:
        raise ValueError("K must be a multiple of 16")
    gs = np.float32(global_scale)
    blocks = x_bits.reshape(M, K // NV_BLOCK, NV_BLOCK)
    mag = bf16_to_f64(blocks & np.uint16(0x7FFF)).astype(np.float32)  # exact
    vmax = mag.max(axis=-1)
    # a binary32 product may overflow to infinity for huge global scales: the E4M3 and E2M1 steps then
    # saturate it, as the conversions do
    with np.errstate(over="ignore"):
        sf = (gs * (vmax * RCP6_F32).astype(np.float32)).astype(np.float32)
    sf_code = e4m3_magnitude_code(sf.astype(np.float64))
    sf_deq = E4M3_MAGNITUDES[sf_code].astype(np.float32)
    with np.errstate(divide="ignore"):
        r = np.where(sf_deq > 0, gs / np.where(sf_deq > 0, sf_deq, np.float32(1)), np.float32(0)).astype(np.float32)
    with np.errstate(over="ignore"):
        v = (mag * r[..., None]).astype(np.float32)
    code = e2m1_magnitude_code(v.astype(np.float64))
    code |= ((blocks >> np.uint16(15)).astype(np.uint8) << np.uint8(3))
    code = code.reshape(M, K)
    q = (code[:, 0::2] | (code[:, 1::2] << np.uint8(4))).astype(np.uint8)
    return q, sf_code.astype(np.uint8)


def nvfp4_dequant_ref(q, scale_codes, global_scale):
    """x_hat = (-1)**s * E2M1 value * SF_deq / global_scale, float64 (SF_deq the E4M3 scale's value)."""
    codes = unpack_codes(q)
    mag = E2M1_MAGNITUDES[codes & 7]
    sign = np.where(codes & 8, -1.0, 1.0)
    s = np.repeat(E4M3_MAGNITUDES[np.asarray(scale_codes, dtype=np.uint8)], NV_BLOCK, axis=-1)
    return sign * mag * s / float(np.float32(global_scale))


def nv_tile_scales(flat):
    """NVFP4 scale bytes [M, K/16] in the same tiled layout as tile_scales (128 rows by 4 scale
    columns per 512-byte tile; reading: the pages' tiling is written for scale columns, whatever the
    block size)."""
    return tile_scales(flat)
