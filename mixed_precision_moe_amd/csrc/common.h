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

