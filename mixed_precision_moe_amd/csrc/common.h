// Device-side definitions shared by the gfx950 MXFP4 / MoE kernels: vector types, the E8M0 rule and
// conversions; the memory layouts the kernels agree on are in layout.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x32_t __attribute__((ext_vector_type(32)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x16_t __attribute__((ext_vector_type(16)));

#define MX_DEV __device__ __forceinline__

// ---------------------------------------------------------------------------------------------
// E8M0 scale of a block from the binary32 bits of its largest magnitude (the 0.75 round-up rule):
// add 2^21 so significands >= 1.75 carry into the next binade, take the biased exponent B,
// e = B - 2 clamped to [0, 254]; a zero maximum gives 0.
// [P3 Implementation breakdown item 1; Key source snippets, the UE8M0_SF branch]
MX_DEV uint32_t e8m0_from_amax_bits(uint32_t amax_bits) {
  uint32_t b = ((amax_bits + (1u << 21)) >> 23) & 0xFFu;
  uint32_t e = b > 2u ? b - 2u : 0u;
  e = e < 254u ? e : 254u;
  return amax_bits == 0u ? 0u : e;
}

// E8M0 scale of an MXFP8 block (E4M3 elements): the same round-up of the block maximum at a
// significand of 1.75, minus E4M3's largest element exponent 8 instead of E2M1's 2, so the maximum maps
// into [224, 448) and no element saturates (448 = 1.75 * 2^8 is E4M3's largest magnitude).
MX_DEV uint32_t e8m0_e4m3_from_amax_bits(uint32_t amax_bits) {
  uint32_t b = ((amax_bits + (1u << 21)) >> 23) & 0xFFu;
  uint32_t e = b > 8u ? b - 8u : 0u;
  e = e < 254u ? e : 254u;
  return amax_bits == 0u ? 0u : e;
}

// The scale operand of the gfx950 scaled conversions: only its exponent field is used, as an E8M0
// exponent (field 0 means 2^-127), so the byte shifted into place is the scale.
MX_DEV float e8m0_as_scale_operand(uint32_t e) { return __uint_as_float(e << 23); }

MX_DEV float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// binary32 -> bf16 bits, round to nearest even (finite inputs).
MX_DEV uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Position p of a 32-element K block of the second GEMM's operands holds element W2_PERM(p) of
// the block: the first GEMM's transposed output leaves lane half h with block elements
// 8*jj + 4*h + i (accumulator index 4*jj + i), which it stores at positions 16*h + 4*jj + i.
__host__ __device__ inline int w2_perm(int p) { return 8 * ((p & 15) >> 2) + 4 * (p >> 4) + (p & 3); }

// Stores the SLOT / 4 words of lane L's operand slot into the region-ordered slots `blk` of its row
// group and K step (slot_byte in layout.h): one 16- or 8-byte store per region, each coalesced over
// the wave.
template <int AF>
MX_DEV void store_slot(uint8_t* blk, int L, const uint32_t* words) {
  constexpr int SLOT = act_slot(AF);
#pragma unroll
  for (int o = 0; o < SLOT; o += 8) {
    if (slot_region_start(AF, o) != o) continue;
    if (slot_region_bytes(AF, o) == 16)
      *reinterpret_cast<u32x4_t*>(blk + slot_byte(AF, L, o)) =
          u32x4_t{words[o / 4], words[o / 4 + 1], words[o / 4 + 2], words[o / 4 + 3]};
    else
      *reinterpret_cast<u32x2_t*>(blk + slot_byte(AF, L, o)) = u32x2_t{words[o / 4], words[o / 4 + 1]};
  }
}

// ---------------------------------------------------------------------------------------------
// Activation split helpers: 32 bf16 of one block held as 16 words (w[j]: elements 2j, 2j + 1).
typedef decltype(__builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(bf16x32_t{}, 1.0f)) fp6x32_t;

MX_DEV uint32_t amax_bits32(const uint32_t* w) {  // 16 words = 32 bf16 -> largest magnitude bits
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 16; i++) m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  return m;
}

typedef short xs16x2_t __attribute__((ext_vector_type(2)));


// The three terms of a bf16 block (w[j]: elements 2j, 2j + 1) into slot[0..15] (E2M3 codes of t0 and
// t1, six dwords each, then the 16 bytes of E2M1 codes of t2, element i at code i), returning the
// scale dword (e0 | e1 << 8 | e2 << 16).  The block is held as its even (ev) and odd (od) elements in
// binary32, where every value involved is exact: a bf16 value, an E2M3 code times its power-of-two
// scale (four significant bits) and each remainder, which is again exact in bf16.  So the split is the
// one bf16 arithmetic gives, with no conversion back to bf16 between the terms.
MX_DEV uint32_t split3_bf16(const uint32_t* w, uint32_t* slot) {
  f32x16_t ev, od;
#pragma unroll
  for (int j = 0; j < 16; j++) {
    ev[j] = __uint_as_float(w[j] << 16);
    od[j] = __uint_as_float(w[j] & 0xFFFF0000u);
  }
  // block maximum of magnitudes (four independent chains) -> E8M0 scale (the 0.75 round-up rule)
  auto scale_of = [&]() __attribute__((always_inline)) {
    float m4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 16; j++) m4[j & 3] = fmaxf(fmaxf(m4[j & 3], fabsf(ev[j])), fabsf(od[j]));
    return e8m0_from_amax_bits(__float_as_uint(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]))));
  };
  uint32_t scales = 0;
#pragma unroll
  for (int term = 0; term < 2; term++) {
    const uint32_t e = scale_of();
    scales |= e << (8 * term);
    const float sv = e8m0_as_scale_operand(e);
    // code 2j <- ev[j], code 2j + 1 <- od[j].  The conversion reads its sources over several passes
    // while it writes its six result registers, so the result must not share a register with a
    // source: the instruction is issued with an early-clobber output.
    fp6x32_t codes;
    asm("v_cvt_scalef32_2xpk16_fp6_f32 %0, %1, %2, %3" : "=&v"(codes) : "v"(ev), "v"(od), "v"(sv));
#pragma unroll
    for (int d = 0; d < 6; d++) slot[6 * term + d] = codes[d];
    // the dequantized term in bf16 (exact), pairs (2j, 2j + 1) per word: half the registers of binary32
    const auto deq = __builtin_bit_cast(u32x16_t, __builtin_amdgcn_cvt_scalef32_pk32_bf16_fp6(codes, sv));
#pragma unroll
    for (int j = 0; j < 16; j++) {
      ev[j] = ev[j] - __uint_as_float(deq[j] << 16);
      od[j] = od[j] - __uint_as_float(deq[j] & 0xFFFF0000u);
    }
  }
  const uint32_t e2 = scale_of();
  const float sv = e8m0_as_scale_operand(e2);
#pragma unroll
  for (int d = 0; d < 4; d++) {
    uint32_t p = 0;
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, ev[4 * d], od[4 * d], sv, 0);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, ev[4 * d + 1], od[4 * d + 1], sv, 1);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, ev[4 * d + 2], od[4 * d + 2], sv, 2);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, ev[4 * d + 3], od[4 * d + 3], sv, 3);
    slot[12 + d] = p;
  }
  return scales | (e2 << 16);
}

// 32 bf16 (w[j]: elements 2j, 2j + 1) -> E2M1 codes, element i in nibble i of the 16 bytes
MX_DEV void fp4_from_bf16(const uint32_t* w, float sc, uint32_t* out) {
#pragma unroll
  for (int d = 0; d < 4; d++) {
    uint32_t p = 0;
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(p, __builtin_bit_cast(bf16x2_t, w[4 * d]), sc, 0);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(p, __builtin_bit_cast(bf16x2_t, w[4 * d + 1]), sc, 1);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(p, __builtin_bit_cast(bf16x2_t, w[4 * d + 2]), sc, 2);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(p, __builtin_bit_cast(bf16x2_t, w[4 * d + 3]), sc, 3);
    out[d] = p;
  }
}

// 32 bf16 -> E4M3 codes, element i in byte i of the 32 bytes
MX_DEV void fp8_from_bf16(const uint32_t* w, float sc, uint32_t* out) {
#pragma unroll
  for (int d = 0; d < 8; d++) {
    xs16x2_t p = xs16x2_t{0, 0};
    p = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(p, __builtin_bit_cast(bf16x2_t, w[2 * d]), sc, false);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(p, __builtin_bit_cast(bf16x2_t, w[2 * d + 1]), sc, true);
    out[d] = __builtin_bit_cast(uint32_t, p);
  }
}
