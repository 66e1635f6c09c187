// Grouped expert GEMMs of the MoE layer on gfx950 block-scaled MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4), with the SwiGLU and the routing-weighted output fused into
// their epilogues, and the final combine over the top-k experts of each token.
//
// [DEF: grouped w13 GEMM, SwiGLU = silu(w1 half) * (w3 half), grouped w2 GEMM, weighted top-k combine;
//  MXFP4 weights with E8M0 scales per 32 elements; P1 Implementation breakdown: the mixed-input fused
//  MoE multiplies packed 4-bit weights with per-32 group scales by 16-bit activations]
//
// The MFMA has no bf16 operand, so a bf16 activation enters as three block-scaled terms x = t0 + t1 + t2
// (E2M3, E2M3 of the remainder, E2M1 of what is left; each with its own E8M0 scale per 32 elements),
// and every product is issued once per term against the same FP4 weight registers; FP6 x FP4 and
// FP4 x FP4 run at the same rate on gfx950.  The first GEMM's output (the SwiGLU activation) stays fp32
// until it is split into the second GEMM's three terms, and the second GEMM's rows are 16-bit integers
// with a power-of-two scale per 16 columns that the combine sums in fp32, so the only bf16 rounding
// after the input is the output's.  The quantized-activation formats (MXFP8, MXFP4) are one term.
//
// Both GEMMs are computed transposed, D[n][m] = sum_k W[n][k] act[m][k]: the weights are the A operand
// (rows n = 32 output columns of one tile), the tokens the B operand (columns m = 32 rows of the padded
// row order).  Lane l of a 32x32 result holds token l%32 and tile rows 8*jj + 4*(l/32) + i.
//  - First GEMM: gate and up of a token sit in the same lane (SwiGLU in registers); the 32-element
//    blocks of two adjacent activation tiles are spread over both lane halves, and one exchange of
//    halves leaves each lane one whole block, which it splits into the second GEMM's operand terms.
//  - Second GEMM: one exchange of halves leaves each lane 16 consecutive output columns of its token,
//    stored as 16-bit integers with one power-of-two exponent per 16 columns (an absolute error of at
//    most 2^-14 of the block maximum) in the padded row order; the combine gathers each token's k rows.
//
// Both GEMMs run one kernel template.  A workgroup of four waves (WR x WC) computes an M tile of
// NRG = WR*RW row groups of 32 rows against NT = WC*CW weight tiles of 32 columns; wave (wr, wc) holds
// RW x CW accumulators.  Per 64-wide K step the workgroup copies the step's operands global -> LDS
// with LDS DMA (global_load_lds: no registers, no address math beyond the source) into a ring of D
// stages: every wave issues the same number of copies per stage, waits for its own with vmcnt and one
// barrier per step publishes the stage.  Operand fragments of step kt+1 are read from LDS while the
// MFMAs of step kt run: a fixed plan (StepPlan) orders each step's MFMAs and puts after each MFMA its
// share of the fragment loads and copies, so their instructions issue while the matrix core works.
// Configurations with a 3-stage ring at two workgroups per CU (the second GEMM, the first GEMM's
// 64-row tiles) instead load step kt+1's fragments after step kt's MFMAs ("late"), which leaves the
// copies about one more step to land.
// Work items (M tile, column position) are dealt to XCDs in contiguous ranges
// so the column positions of one M tile (same gathered tokens) and consecutive tiles of one expert
// (same weights) share an XCD's L2.
#pragma once

#include <type_traits>

#include "common.h"
#include "internal.h"

namespace {

typedef __attribute__((address_space(3))) void* lds_vptr_t;

constexpr int kXcds = 8;           // workgroup b runs on XCD b % 8
constexpr int kBufFlags = 0x00020000;  // buffer resource word 3: raw dword access (stride 0)


// LDS DMA: lane i copies 16 (or 4) bytes from its global address to lds_wave_base + i * 16 (or 4).
// (Sub-dword copies still occupy a dword per lane in LDS, so every copied record here is a dword or
// a multiple of 16 bytes.)  The copies are issued as inline assembly with M0 set explicitly: the
// compiler's wait-count tracking treats its own global_load_lds as a FLAT access to both memories and
// would then wait for every LDS load (lgkmcnt(0)) before any use of one.  Every wait for these copies
// is therefore explicit (vmcnt, counted per stage) and each LDS consumer follows such a wait and a
// barrier.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is listed as clobbered; nothing else here uses it
// lds_wave_base is an LDS byte address, uniform over the wave (it goes to M0).
MX_DEV void dma16(const void* g, uint32_t lds_wave_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_wave_base);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "s"(m0) : "memory", "m0");
}
MX_DEV void dma4(const void* g, uint32_t lds_wave_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_wave_base);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" : : "v"(g), "s"(m0) : "memory", "m0");
}
#pragma clang diagnostic pop

// f(integral_constant<int, i>) for i = 0 .. N-1 (operand selectors of the MFMA must be literals).
template <int I, int N, typename F>
MX_DEV void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

template <int N>
MX_DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x70 | 0xF00);
}
MX_DEV void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Barrier without the implied full vmcnt wait of __syncthreads: the LDS DMA copies are waited for
// explicitly, so only LDS and compiler ordering are needed here.
MX_DEV void block_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Reads an accumulator element where the epilogue needs it: the operand stays in its AGPR until this
// point, so the accumulator tiles are not all copied to VGPRs when the K loop ends.
MX_DEV float acc_read(float v) {
  float r;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(v));
  return r;
}

// ------------------------------------------------------------------------------------------------
// Kernel configuration.  LDS stage: [NT weight pieces of 1 KB][1 KB weight scale records of the
// column block], then the activation: first GEMM [NRG row groups x 32 rows x REC-byte records]
// (padded to whole 1 KB copies); second GEMM [NRG x 64 lanes x SLOT-byte activation slots]
// [NRG x 256 B activation scale dwords].
template <bool G1, int AF, int WR, int WC, int RW, int CW, int D>
struct Cfg {
  static constexpr int NRG = WR * RW, NT = WC * CW;
  static_assert(WR * WC == 4, "four waves");
  static_assert(NT == 8 || NT == 16, "a workgroup covers a column block or half of one");
  static_assert(CW % 4 == 0, "weight scales are read four tiles per dword");
  static_assert(D >= 3 && D <= 6, "ring depth");  // stages issued D - 1 steps ahead
  static constexpr int SLOT = act_slot(AF), REC = act_rec(AF), NTERMS = act_terms(AF);
  static constexpr int CH = REC / 16;              // 16-byte chunks of a first-GEMM record
  static constexpr int kRecChunks = 32 * CH;       // ... of the records of one row group
  static constexpr int kXRG = 64 * SLOT;           // second GEMM: activation bytes of one row group
  static constexpr int kXBytes = G1 ? (NRG * kRecChunks * 16 + 1023) / 1024 * 1024 : NRG * kXRG;
  static constexpr int oW = 0, oWS = NT * 1024, oX = oWS + 1024, oXS = oX + kXBytes;
  static constexpr int kStage = oXS + (G1 ? 0 : NRG * 256);
  static constexpr int nW = NT / 4;                // weight pieces copied per wave
  static constexpr int nXI = kXBytes / 1024;       // 1 KB activation copies per stage
  static constexpr int nX = (nXI + 3) / 4;         // ... per wave (the last one repeated)
  static constexpr int nXS = G1 ? 0 : (NRG + 3) / 4;  // activation scale copies per wave
  static constexpr int kOps = nW + 1 + nX + nXS;   // copies per wave per stage
};

// LDS of one workgroup: the ring, then the per-item tables (double-buffered by item parity): the first
// GEMM's row tokens and, with biases, the gate / up bias entries; the second GEMM's row weights and biases.
template <bool G1, int AF, bool BIAS, int WR, int WC, int RW, int CW, int D>
struct Lds {
  using C = Cfg<G1, AF, WR, WC, RW, CW, D>;
  static constexpr int kTab = C::NRG * 32 > 64 ? C::NRG * 32 : 64;  // row table entries (one dword copy covers 64)
  static constexpr int kBias = G1 ? C::NT / 2 * 32 : C::NT * 32;   // bias entries of one half (first GEMM) or of the tile
  static constexpr int kTabRow = 2 * kTab * 4, kTabB = BIAS ? 2 * (G1 ? 2 : 1) * kBias * 2 : 0;
  static constexpr int kBytes = D * C::kStage + kTabRow + kTabB;
  // two workgroups per CU where both fit in its 160 KB
  static constexpr int kOcc = 2 * kBytes <= 160 * 1024 ? 2 : 1;
};

// Order of the work of one K step of a wave: its NM MFMAs in a fixed order (groups of two weight
// tiles, PG = 2 * NTERMS * RW MFMAs each; within a group term-major, then row group, then tile, so an
// accumulator is reused 2 * RW MFMAs later), and after MFMA m up to kCap of the other tasks of the
// step, so that their instructions issue while the matrix core works:
//   kDef + i : weight fragment CW - 2 + i of this step, from the current stage (the last group's
//              fragments are reloaded at the start of the step that uses them)
//   kX + r   : activation fragments and scale of row group r for the next step, from the next stage
//   kWs      : weight scale dwords for the next step
//   kRel + j : weight fragment j (< CW - 2) for the next step, after the last MFMA that uses it
//   kDma + i : copy i of the stage D - 1 steps ahead
struct StepTask {
  static constexpr int kNone = -1, kDef = 0, kX = 10, kWs = 20, kRel = 30, kDma = 100;
};
// COPIES_FIRST puts the copies right after the step's first MFMAs (for a latency-bound GEMM with few
// K steps per item); otherwise they are spread over the MFMAs after the first group.
// LATE: the step's fragment loads are not interleaved (they follow the step's MFMAs, see the kernel);
// only the copies are placed.
template <int RW, int CW, int KOPS, bool COPIES_FIRST, bool LATE, int NTERMS>
struct StepPlan {
  static constexpr int G = CW / 2, PG = 2 * NTERMS * RW, NM = PG * G, kCap = 6;
  static constexpr int kTasks = LATE ? KOPS : 2 + RW + 1 + (CW - 2) + KOPS;
  // tasks after one MFMA before later MFMAs take them: 2, or more when a step has few MFMAs
  static constexpr int kPer = (kTasks + NM - 1) / NM > 2 ? (kTasks + NM - 1) / NM : 2;
  int t[NM][kCap];
  constexpr void place(int task, int earliest) {
    int m = earliest < NM ? earliest : NM - 1;
    while (m < NM - 1 && n_at(m) >= kPer) m++;
    int c = n_at(m);
    t[m][c < kCap ? c : kCap - 1] = task;
  }
  constexpr int n_at(int m) const {
    int c = 0;
    while (c < kCap && t[m][c] != StepTask::kNone) c++;
    return c;
  }
  constexpr StepPlan() : t{} {
    for (int m = 0; m < NM; m++)
      for (int c = 0; c < kCap; c++) t[m][c] = StepTask::kNone;
    if (LATE) {
      for (int i = 0; i < KOPS; i++) place(StepTask::kDma + i, COPIES_FIRST ? 0 : i * NM / KOPS);
      return;
    }
    // the last group's fragments shortly before that group, so few loads are younger than them
    const int def_at = (G - 1) * PG - 4 > 0 ? (G - 1) * PG - 4 : 0;
    if (COPIES_FIRST) {
      place(StepTask::kDef + 0, def_at);
      place(StepTask::kDef + 1, def_at);
      for (int i = 0; i < KOPS; i++) place(StepTask::kDma + i, 0);
    }
    for (int r = 0; r < RW; r++) place(StepTask::kX + r, 0);
    place(StepTask::kWs, 0);
    for (int j = 0; j < CW - 2; j++) place(StepTask::kRel + j, (j / 2 + 1) * PG - 1);
    if (!COPIES_FIRST) {
      for (int i = 0; i < KOPS; i++) place(StepTask::kDma + i, PG + i * (NM - PG) / KOPS);
      place(StepTask::kDef + 0, def_at);
      place(StepTask::kDef + 1, def_at);
    }
  }
  // every task placed exactly once, the last group's fragments before that group
  constexpr bool valid() const {
    int n = 0, def_last = 0;
    for (int m = 0; m < NM; m++)
      for (int c = 0; c < kCap; c++)
        if (t[m][c] != StepTask::kNone) {
          n++;
          if (t[m][c] < StepTask::kX) def_last = m;
        }
    if (LATE) return n == KOPS && n_at(NM - 1) < kCap;
    return n == 2 + RW + 1 + (CW - 2) + KOPS && def_last < (G - 1) * PG && n_at(NM - 1) < kCap;
  }
};


typedef const __attribute__((address_space(3))) uint16_t lds_u16;
typedef const __attribute__((address_space(3))) uint8_t* lds_u8;

// Exchanges lane halves: returns {lanes 0-31 of x, then lanes 0-31 of y} and {lanes 32-63 of x, then
// lanes 32-63 of y} (one v_permlane32_swap).
MX_DEV void swap_halves(float& x, float& y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, y), false,
                                                  false);
  x = __builtin_bit_cast(float, (unsigned)r[0]);
  y = __builtin_bit_cast(float, (unsigned)r[1]);
}

MX_DEV void swap_halves_u32(uint32_t& x, uint32_t& y) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, y, false, false);
  x = (uint32_t)r[0];
  y = (uint32_t)r[1];
}

// Four consecutive bf16 entries of an LDS bias table (8-byte aligned) as fp32.
MX_DEV void bias4(lds_u16* p, float* out) {
  const u32x2_t v = *reinterpret_cast<const __attribute__((address_space(3))) u32x2_t*>(p);
  out[0] = __uint_as_float(v[0] << 16);
  out[1] = __uint_as_float(v[0] & 0xFFFF0000u);
  out[2] = __uint_as_float(v[1] << 16);
  out[3] = __uint_as_float(v[1] & 0xFFFF0000u);
}

typedef short g1s16x2_t __attribute__((ext_vector_type(2)));

// E8M0 scale (the 0.75 round-up rule) of the block lo[0..15], hi[0..15] (positions q and 16 + q),
// also put into byte `term` of `scales`: the block maximum of magnitudes in four independent chains of
// three-operand maxima.
MX_DEV uint32_t block_amax_e8m0(const float* lo, const float* hi, uint32_t& scales, int term) {
  float m4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < 16; q += 2) {
    m4[(q / 2) & 1] = fmaxf(fmaxf(m4[(q / 2) & 1], fabsf(lo[q])), fabsf(lo[q + 1]));
    m4[2 + ((q / 2) & 1)] = fmaxf(fmaxf(m4[2 + ((q / 2) & 1)], fabsf(hi[q])), fabsf(hi[q + 1]));
  }
  const float amax = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
  const uint32_t ex = e8m0_from_amax_bits(__float_as_uint(amax));
  scales |= ex << (8 * term);
  return ex;
}

// The block lo, hi (positions q, 16 + q) as E2M1 codes, position p in nibble p of the 16 bytes.
MX_DEV void fp4_from_f32(const float* lo, const float* hi, float sv, uint32_t* out) {
#pragma unroll
  for (int d = 0; d < 4; d++) {
    const float* src = d < 2 ? lo + 8 * d : hi + 8 * (d - 2);
    uint32_t p = 0;
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, src[0], src[1], sv, 0);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, src[2], src[3], sv, 1);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, src[4], src[5], sv, 2);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, src[6], src[7], sv, 3);
    out[d] = p;
  }
}

// First GEMM epilogue for the activation tiles `it` (even) and it + 1 of one row group, which together
// are one K step (kt2 = it / 2) of the second GEMM: bias, SwiGLU in fp32, then one exchange of lane
// halves after which lane l holds the whole 32-element block of token l % 32 in tile it + l / 32,
// converted to the terms of activation format AF and written as one operand slot of the second GEMM
// (lane l of the step) and its scale dword.  When tile it + 1 is past I / 32 its half is a zero block.
// g0/u0, g1/u1: gate and up accumulators of the two tiles; bg/bu: the 64 gate / up biases of the pair
// (bf16, LDS), read when BIAS.  SECOND is false only for the last pair of an odd tile count.
template <bool BIAS, bool SECOND, int AF>
MX_DEV void g1_epilogue_pair(const f32x16_t& g0, const f32x16_t& u0, const f32x16_t& g1, const f32x16_t& u1,
                             const GemmArgs& a, lds_u16* bg, lds_u16* bu, int kt2, int rg, int lane) {
  const int h = lane >> 5;
  // All 64 accumulator values are read first: each read is a volatile asm statement, which the
  // scheduler treats as a region boundary, so reading them up front leaves the SwiGLU arithmetic of the
  // whole pair as one region whose 32 independent exp / reciprocal chains can interleave.
  float ra[4][16];
#pragma unroll
  for (int q = 0; q < 16; q++) {
    ra[0][q] = acc_read(g0[q]);
    ra[1][q] = acc_read(u0[q]);
    ra[2][q] = acc_read(g1[q]);
    ra[3][q] = acc_read(u1[q]);
  }
  // lo[q], hi[q]: block positions q and 16 + q after the exchange (position p of a block holds the
  // tile's row 8 * ((p & 15) >> 2) + 4 * (p >> 4) + (p & 3), the order the second GEMM's weights use)
  float lo[16], hi[16];
#pragma unroll
  for (int jj = 0; jj < 4; jj++) {
    // accumulator 4*jj + i holds row 8*jj + 4*h + i of its tile: four consecutive bias entries
    float b1a[4] = {0.f, 0.f, 0.f, 0.f}, b3a[4] = {0.f, 0.f, 0.f, 0.f};
    float b1b[4] = {0.f, 0.f, 0.f, 0.f}, b3b[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (BIAS) {
      const int o = 8 * jj + 4 * h;
      bias4(bg + o, b1a);
      bias4(bu + o, b3a);
      bias4(bg + 32 + o, b1b);
      bias4(bu + 32 + o, b3b);
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int q = 4 * jj + i;
      // silu(g) = g / (1 + exp(-g)) with the hardware exponential and reciprocal (exp overflow gives 0);
      // without biases nothing is added (x + 0 is not foldable: it turns -0 into +0)
      float ga = ra[0][q], ua = ra[1][q], gb = ra[2][q], ub = ra[3][q];
      if constexpr (BIAS) {
        ga += b1a[i];
        ua += b3a[i];
        gb += b1b[i];
        ub += b3b[i];
      }
      float va = ga * __builtin_amdgcn_rcpf(1.0f + __expf(-ga)) * ua;
      float vb = gb * __builtin_amdgcn_rcpf(1.0f + __expf(-gb)) * ub;
      if constexpr (!SECOND) vb = 0.f;
      swap_halves(va, vb);
      lo[q] = va;
      hi[q] = vb;
    }
  }
  constexpr int SLOT = act_slot(AF);
  const int64_t blk = (int64_t)rg * a.nkt2 + kt2;
  uint32_t out[SLOT / 4];
  uint32_t scales = 0;
  if constexpr (AF == kActBf16) {
    // Terms 0 and 1 are the fp32 remainder rounded to E2M3 (nearest even) under its block's scale;
    // term 2 rounds what is left to E2M1.  The fp32-input E2M3 conversion takes the block's even
    // positions from its first source and the odd ones from its second (code 2j <- ev[j], code 2j + 1
    // <- od[j]).
#pragma unroll
    for (int term = 0; term < 2; term++) {
      const float sv = e8m0_as_scale_operand(block_amax_e8m0(lo, hi, scales, term));
      f32x16_t ev, od;
#pragma unroll
      for (int q = 0; q < 16; q += 2) {
        ev[q / 2] = lo[q];
        od[q / 2] = lo[q + 1];
        ev[8 + q / 2] = hi[q];
        od[8 + q / 2] = hi[q + 1];
      }
      // The conversion reads its sources over several passes while it writes its six result
      // registers, so the result must not share a register with any source; the builtin carries no
      // such constraint (the compiler gave the result the scale operand's register, which corrupted the
      // codes), so the instruction is issued with an early-clobber output.
      fp6x32_t codes;
      asm("v_cvt_scalef32_2xpk16_fp6_f32 %0, %1, %2, %3" : "=&v"(codes) : "v"(ev), "v"(od), "v"(sv));
#pragma unroll
      for (int d = 0; d < 6; d++) out[term * 6 + d] = codes[d];
      const auto deq = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(codes, sv);
#pragma unroll
      for (int q = 0; q < 16; q++) {
        lo[q] = lo[q] - deq[q];
        hi[q] = hi[q] - deq[16 + q];
      }
    }
    fp4_from_f32(lo, hi, e8m0_as_scale_operand(block_amax_e8m0(lo, hi, scales, 2)), out + 12);
  } else if constexpr (AF == kActMxfp8) {
    float amax = 0.f;
#pragma unroll
    for (int q = 0; q < 16; q++) amax = fmaxf(amax, fmaxf(fabsf(lo[q]), fabsf(hi[q])));
    const uint32_t ex = e8m0_e4m3_from_amax_bits(__float_as_uint(amax));
    scales = ex;
    const float sv = e8m0_as_scale_operand(ex);
#pragma unroll
    for (int d = 0; d < 8; d++) {
      // positions 4d .. 4d + 3: two pairs, one per 16-bit half
      const float* src = d < 4 ? lo + 4 * d : hi + 4 * (d - 4);
      g1s16x2_t p = g1s16x2_t{0, 0};
      p = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(p, src[0], src[1], sv, false);
      p = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(p, src[2], src[3], sv, true);
      out[d] = __builtin_bit_cast(uint32_t, p);
    }
  } else {
    fp4_from_f32(lo, hi, e8m0_as_scale_operand(block_amax_e8m0(lo, hi, scales, 0)), out);
  }
  store_slot<AF>(a.actq + blk * 64 * SLOT, lane, out);
  reinterpret_cast<uint32_t*>(a.acts)[blk * 64 + lane] = scales;
}

// ------------------------------------------------------------------------------------------------
// The grouped GEMM.  G1: first GEMM (A = weights, B = gathered token terms, SwiGLU epilogue);
// otherwise the second GEMM (A = weights, B = activation terms, weighted 16-bit rows to o16).
//
// A workgroup processes the items (M tile, column position) dealt to it in turn; the first D - 1
// stages of the next item are copied before the current item's epilogue runs, so the ring refills
// while the epilogue computes and stores.  The first GEMM gathers the next item's token rows through a
// table of its token indices, which one copy per wave brings into LDS at the start of the current item.
template <int NX, int NXS>
struct ItemSrc {
  int prow0, nrows; // the item's tile: first padded row and rows of its expert (read with the sources)
  int64_t wb;       // byte offset of this wave's first weight piece of step 0 (uniform)
  int64_t wsb;      // byte offset of this wave's quarter of the step-0 scale records (uniform)
  uint32_t x[NX];   // byte offsets of this lane's activation copies of step 0
  uint32_t xs[NXS > 0 ? NXS : 1]; // byte offsets of this lane's activation scale copies of step 0
};

template <bool G1, int AF, bool BIAS, int WR, int WC, int RW, int CW, int D, int OCC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(OCC))) void grouped_gemm_kernel(GemmArgs a) {
  using C = Cfg<G1, AF, WR, WC, RW, CW, D>;
  constexpr int NRG = C::NRG, NT = C::NT, NTERMS = C::NTERMS;
  using L = Lds<G1, AF, BIAS, WR, WC, RW, CW, D>;
  constexpr int kTab = L::kTab, kBias = L::kBias, kTabRow = L::kTabRow;
  static_assert(L::kBytes * OCC <= 160 * 1024, "LDS of OCC workgroups per CU");
  // The ring and the per-item tables (copied with LDS DMA one item ahead) in one LDS object, so the
  // compiler's tracking of LDS DMA writes sees a single buffer.
  __shared__ __attribute__((aligned(16))) uint8_t smem[L::kBytes];
  int32_t(*t_row)[kTab] = reinterpret_cast<int32_t(*)[kTab]>(smem + D * C::kStage);
  uint16_t(*t_b)[G1 ? 2 : 1][kBias] = reinterpret_cast<uint16_t(*)[G1 ? 2 : 1][kBias]>(smem + D * C::kStage + kTabRow);
  const int tid = threadIdx.x;
  // LDS byte address of smem (address-space arithmetic from here on, no generic-pointer conversions)
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(lds_vptr_t)smem;
  const int nkt = a.nkt, ncb = a.ncb;
  const int nx = ncb * kCB / NT;
  const int nrec = a.nrec;  // K-step records per token row of xq (first GEMM)

  const int total = *a.ntiles * nx;
  const int chunk = (total + kXcds - 1) / kXcds;
  const int xcd = blockIdx.x % kXcds, per_xcd = gridDim.x / kXcds;
  const int p0 = blockIdx.x / kXcds;
  // items of this workgroup: q = 0 .. nq - 1 -> item xcd * chunk + p0 + q * per_xcd
  int nq = 0;
  if (p0 < chunk) {
    const int last = min(chunk, total - xcd * chunk);  // local positions of this XCD's items
    if (last > p0) nq = (last - p0 + per_xcd - 1) / per_xcd;
  }
  if (nq == 0) return;

  int lane, wave;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
  asm volatile("s_lshr_b32 %0, %1, 6" : "=s"(wave) : "s"(__builtin_amdgcn_readfirstlane(tid)));
  const int wr = wave / WC, wc = wave % WC;

  auto item_of = [&](int q) __attribute__((always_inline)) { return xcd * chunk + p0 + q * per_xcd; };

  // Copy sources of an item.  G1 takes the tokens of the item's rows from `tab` (LDS) when given, else
  // from global memory.
  using Src = ItemSrc<C::nX, C::nXS>;
  auto make_src = [&](int item, int tb, Src& sr) __attribute__((always_inline)) {
    const int tile = item / nx, x = item % nx;
    const TileDesc td = a.tiles[tile];
    const int e = td.e, prow0 = td.prow0;
    sr.prow0 = prow0;
    sr.nrows = td.nrows;
    const int cb = x * NT / kCB, jj0 = (x * NT) % kCB;
    const int64_t wstep0 = (int64_t)(e * ncb + cb) * nkt;
    sr.wb = wstep0 * (kCB * 1024) + (jj0 + wave * C::nW) * 1024;
    sr.wsb = wstep0 * 1024 + wave * 256;
#pragma unroll
    for (int q = 0; q < C::nX; q++) {
      int o = wave + 4 * q;
      o = o < C::nXI ? o : C::nXI - 1;
      if (G1) {
        // 16-byte chunk c of the stage's records: row c / 7 of the tile, part c % 7 of its record; the
        // chunks past the last row (one row group) repeat the last chunk into the stage's padding
        int c = o * 64 + lane;
        c = c < NRG * C::kRecChunks ? c : NRG * C::kRecChunks - 1;
        const int row = c / C::CH, part = c % C::CH;
        const int tok = tb >= 0 ? t_row[tb][row] : a.prow_tok[prow0 + row];
        sr.x[q] = (uint32_t)(tok * nrec * C::REC + part * 16);
      } else {
        constexpr int per_rg = C::kXRG / 1024;  // 1 KB copies per row group
        const int rg = o / per_rg, pp = o % per_rg;
        sr.x[q] = (uint32_t)(((prow0 >> 5) + rg) * nkt * C::kXRG + (pp * 64 + lane) * 16);
      }
    }
#pragma unroll
    for (int q = 0; q < C::nXS; q++) {  // second GEMM only
      int o = wave + 4 * q;
      o = o < NRG ? o : NRG - 1;
      sr.xs[q] = (uint32_t)(((prow0 >> 5) + o) * nkt * 256 + lane * 4);
    }
  };
  constexpr int xstep = G1 ? C::REC : C::kXRG;    // bytes per K step of an activation copy
  constexpr int xsstep = 256;                      // ... of an activation scale copy (second GEMM)
  // Copy i (of kOps per wave) of stage `kt` of the item with sources `sr` into ring slot `slot`.
  auto issue_op = [&](const Src& sr, int kt, int slot, auto ic) __attribute__((always_inline)) {
    constexpr int i = decltype(ic)::value;
    const uint32_t base = smem_lds + slot * C::kStage;
    if constexpr (i < C::nW) {
      dma16(a.wq + (sr.wb + kt * (kCB * 1024) + i * 1024) + lane * 16, base + C::oW + (wave * C::nW + i) * 1024);
    } else if constexpr (i == C::nW) {
      dma4(a.ws + (sr.wsb + kt * 1024) + lane * 4, base + C::oWS + wave * 256);
    } else if constexpr (i < C::nW + 1 + C::nX) {
      constexpr int q = i - C::nW - 1;
      int o = wave + 4 * q;
      o = o < C::nXI ? o : C::nXI - 1;
      dma16(a.xq + (sr.x[q] + (uint32_t)(kt * xstep)), base + C::oX + o * 1024);
    } else {
      constexpr int q = i - C::nW - 1 - C::nX;
      int o = wave + 4 * q;
      o = o < NRG ? o : NRG - 1;
      dma4(a.xs + (sr.xs[q] + (uint32_t)(kt * xsstep)), base + C::oXS + o * 256);
    }
  };
  auto issue = [&](const Src& sr, int kt, int slot) __attribute__((always_inline)) {
    static_for<0, C::kOps>([&](auto ic) __attribute__((always_inline)) { issue_op(sr, kt, slot, ic); });
  };
  // The tables of item `item` into buffer `tb`: rows (tokens or weights, kTab dwords) and, with biases,
  // the item's bias entries; 256-byte dword copies spread over the waves (repeats are harmless).
  auto issue_tab = [&](int item, int tb) __attribute__((always_inline)) {
    const int tile = item / nx, x = item % nx;
    const TileDesc td = a.tiles[tile];
    const int prow0 = td.prow0;
    constexpr int kRowOps = kTab / 64;
    const uint8_t* rsrc = G1 ? reinterpret_cast<const uint8_t*>(a.prow_tok) : reinterpret_cast<const uint8_t*>(a.prow_w);
    {
      const int o = wave < kRowOps ? wave : 0;
      dma4(rsrc + (int64_t)(prow0 + o * 64) * 4 + lane * 4, smem_lds + D * C::kStage + (tb * kTab + o * 64) * 4);
    }
    if constexpr (BIAS) {
      constexpr int kBOps = kBias * 2 / 256;  // copies per bias half
      // entries past the end of the bias row (columns beyond I or H, never used) re-read its last pair
      const int len = G1 ? a.I : a.H;
      const uint16_t* brow = a.bias + (int64_t)td.e * (G1 ? 2 * a.I : a.H);
#pragma unroll
      for (int i = 0; i < (G1 ? 2 : 1) * kBOps; i += 4) {
        int o = wave + i;
        o = o < (G1 ? 2 : 1) * kBOps ? o : (G1 ? 2 : 1) * kBOps - 1;
        const int half = o / kBOps, part = o % kBOps;
        int el = x * kBias + part * 128 + lane * 2;  // first of this lane's two entries
        el = el < len - 2 ? el : len - 2;
        dma4(brow + half * len + el,
             smem_lds + D * C::kStage + kTabRow + ((tb * (G1 ? 2 : 1) + half) * kBias) * 2 + part * 256);
      }
    }
  };

  // Each E2M3 term operand (6 dwords) is read by its own two LDS loads (16 + 8 bytes for term 0 at
  // slot offset 0, 8 + 16 bytes for term 1 at offset 24), so every MFMA operand tuple is written in
  // place by its loads.  Each row group's and each term's loads take their base address through an
  // opaque copy: that keeps the compiler from merging adjacent 8-byte loads (of two terms, or of
  // two row groups) into wider loads whose parts would then have to be copied (and waited for) to
  // form the tuples.  Activation fragments and
  // weight scales are double-buffered across steps ([P], P a compile-time parity); a weight fragment
  // is reloaded for the next step after the last MFMA that uses it.
  typedef const __attribute__((address_space(3))) u32x4_t* lds16_p;
  typedef const __attribute__((address_space(3))) u32x2_t* lds8_p;
  typedef const __attribute__((address_space(3))) uint32_t* lds4_p;
  // The 3-stage configurations of the second GEMM (two workgroups per CU) and the first GEMM's 64-row
  // one load the next step's fragments after the step's MFMAs (LATE), so a stage is needed one step
  // later than with loads interleaved into the MFMAs: its copies get about two steps instead of one to
  // land.  The first GEMM's 32-row (decode) configuration and the 128-row ones of both GEMMs measured
  // faster with interleaved loads.
  constexpr bool LATE = D == 3 && (!G1 || RW == 2);
  using Plan = StepPlan<RW, CW, C::kOps, !G1, LATE, NTERMS>;
  static constexpr Plan plan{};
  static_assert(plan.valid(), "step plan");
  // Fragments of the current and the next step: double-buffered by step parity when the next step's
  // loads are interleaved with this step's MFMAs; one buffer in LATE mode, whose loads follow the MFMAs
  // that read the registers (which keeps the two-workgroup configurations within their registers).
  constexpr int NBUF = LATE ? 1 : 2;
  i32x8_t xop[NBUF][RW][NTERMS];
  uint32_t xsc[NBUF][RW];
  u32x4_t w[CW];
  uint32_t wsc[NBUF][CW / 4];
  f32x16_t acc[RW][CW];
  int jj0 = 0;
  auto load_x = [&](const uint8_t* base, int r, auto pc) __attribute__((always_inline)) {
    constexpr int P = LATE ? 0 : decltype(pc)::value;
    // first GEMM: lane l takes block l / 32 of row l % 32's record; second: slot l of the row group
    lds_u8 rec = (lds_u8)(base + C::oX + (wr + WR * r) * (32 * C::REC) + (lane & 31) * C::REC);
    lds_u8 rgb = (lds_u8)(base + C::oX + (wr + WR * r) * C::kXRG);  // second GEMM: the row group's slots
    // Byte O of this lane's slot: in its record (first GEMM), or in the region order of the row group's
    // slots (second GEMM: region [R, R + n) of slot L at 64 * R + n * L)
    auto at = [&](auto oc) __attribute__((always_inline)) {
      constexpr int O = decltype(oc)::value;
      return G1 ? rec + (lane >> 5) * C::SLOT + O : rgb + slot_byte(AF, 0, O) + slot_region_bytes(AF, O) * lane;
    };
    static_for<0, NTERMS>([&](auto tc) __attribute__((always_inline)) {
      constexpr int t = decltype(tc)::value;
      constexpr int off = act_term_offset(AF, t), nb = fmt_bytes(act_term_fmt(AF, t));
      if constexpr (nb == 24) {  // E2M3: 16 + 8 bytes at a 16-byte boundary, else 8 + 16
        constexpr int first = off % 16 == 0 ? 16 : 8;
        lds_u8 pa = at(std::integral_constant<int, off>{});
        asm("" : "+v"(pa));
        lds_u8 pb = at(std::integral_constant<int, off + first>{});
        asm("" : "+v"(pb));
        if constexpr (first == 16) {
          const u32x4_t p4 = *(lds16_p)pa;
          const u32x2_t p2 = *(lds8_p)pb;
          xop[P][r][t] = i32x8_t{(int)p4[0], (int)p4[1], (int)p4[2], (int)p4[3], (int)p2[0], (int)p2[1], 0, 0};
        } else {
          const u32x2_t p2 = *(lds8_p)pa;
          const u32x4_t p4 = *(lds16_p)pb;
          xop[P][r][t] = i32x8_t{(int)p2[0], (int)p2[1], (int)p4[0], (int)p4[1], (int)p4[2], (int)p4[3], 0, 0};
        }
      } else if constexpr (nb == 32) {
        // E4M3: the operand interleaves K by 16: lane half h holds elements 16h .. 16h + 15 of the step's
        // first block, then the same elements of its second block (the scale of block b still comes
        // from lane half b); the two blocks of row l % 32 are the two slots of its record (first GEMM)
        // or the slots of lanes l % 32 and l % 32 + 32 (second GEMM)
        // (second GEMM: the two 16-byte halves are regions at 64 * off and 64 * (off + 16))
        lds_u8 s0 = G1 ? rec + off + (lane >> 5) * 16 : rgb + 64 * off + (lane >> 5) * (64 * 16) + (lane & 31) * 16;
        lds_u8 s1 = s0 + (G1 ? C::SLOT : 32 * 16);
        asm("" : "+v"(s1));
        const u32x4_t p4 = *(lds16_p)s0;
        const u32x4_t q4 = *(lds16_p)s1;
        xop[P][r][t] = i32x8_t{(int)p4[0], (int)p4[1], (int)p4[2], (int)p4[3], (int)q4[0], (int)q4[1], (int)q4[2], (int)q4[3]};
      } else {  // E2M1
        lds_u8 tp = at(std::integral_constant<int, off>{});
        asm("" : "+v"(tp));
        const u32x4_t p4 = *(lds16_p)tp;
        xop[P][r][t] = i32x8_t{(int)p4[0], (int)p4[1], (int)p4[2], (int)p4[3], 0, 0, 0, 0};
      }
    });
    if constexpr (G1)
      xsc[P][r] = *(lds4_p)(rec + 2 * C::SLOT + (lane >> 5) * 4);
    else
      xsc[P][r] = *(lds4_p)(lds_u8)(base + C::oXS + (wr + WR * r) * 256 + lane * 4);
  };
  auto load_w = [&](const uint8_t* base, int j) __attribute__((always_inline)) {
    w[j] = *(lds16_p)(lds_u8)(base + C::oW + (wc * CW + j) * 1024 + lane * 16);
  };
  auto load_ws = [&](const uint8_t* base, auto pc) __attribute__((always_inline)) {
    constexpr int P = LATE ? 0 : decltype(pc)::value;
#pragma unroll
    for (int j4 = 0; j4 < CW / 4; j4++)
      wsc[P][j4] = *(lds4_p)(lds_u8)(base + C::oWS + lane * 16 + jj0 + wc * CW + j4 * 4);
  };

  // MFMA m of a step (the order of StepPlan).  Each is pinned by an ordered use of its accumulator:
  // the MFMAs are pure, and the compiler would otherwise sink them past later waits and barriers
  // (across basic blocks, where scheduling barriers do not reach).
  auto mfma_one = [&](auto mc, auto pc, auto rac) __attribute__((always_inline)) {
    constexpr int m = decltype(mc)::value, P = LATE ? 0 : decltype(pc)::value;
    constexpr int g = m / Plan::PG, u = m % Plan::PG;
    constexpr int t = u / (2 * RW), r = (u % (2 * RW)) / 2, j = 2 * g + (u % 2);
    constexpr int BFMT = act_term_fmt(AF, t);
    if constexpr (r >= decltype(rac)::value) return;  // a row group of padding rows only
    const i32x8_t wo = i32x8_t{(int)w[j][0], (int)w[j][1], (int)w[j][2], (int)w[j][3], 0, 0, 0, 0};
    acc[r][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wo, xop[P][r][t], acc[r][j], kFmtFp4, BFMT, j & 3,
                                                                wsc[P][j >> 2], t, xsc[P][r]);
    asm volatile("" : "+a"(acc[r][j]));
  };

  // Waits until at most n (0 <= n <= N) of this wave's most recent stages may still be in flight
  // (younger copies and stores count too, which only makes the wait longer).
  auto wait_stages = [&](int n, auto nc) __attribute__((always_inline)) {
    constexpr int N = decltype(nc)::value;
    if (n < 0) n = 0;
    if (n >= N) {
      wait_vmcnt<C::kOps * N>();
    } else {
      static_for<0, N>([&](auto ic) __attribute__((always_inline)) {
        if (n == decltype(ic)::value) wait_vmcnt<C::kOps * decltype(ic)::value>();
      });
    }
  };

  Src cur;
  int q = 0;
  int item = item_of(0);
  make_src(item, -1, cur);
  issue_tab(item, 0);
  wait_vmcnt<0>();
  block_sync();
#pragma unroll
  for (int s = 0; s < D - 1; s++)
    if (s < nkt) issue(cur, s, s);

  while (true) {
    const int x = item % nx;
    const int prow0 = cur.prow0, nrows = cur.nrows;  // cur is rebuilt for the next item before the epilogue
    jj0 = (x * NT) % kCB;
    const bool has_next = q + 1 < nq;
    const int tb = q & 1;

    // stage 0 visible: the later stages of the prologue (and younger stores) may be in flight; after
    // the barrier every wave is done with the previous item's tables, so the next item's tables can
    // go to the other buffer.
    wait_stages(nkt - 1, std::integral_constant<int, D - 2>{});
    block_sync();
    if (has_next) issue_tab(item_of(q + 1), tb ^ 1);
    // The K loop for this wave's RA row groups that hold pairs (row group wr + WR r, r < RA; the rest
    // hold padding rows only and get no MFMAs and no fragment loads): every wave issues the same
    // copies and barriers whatever its RA.
    static_assert(RW == 1 || RW == 2, "one or two row groups per wave");
    auto kloop = [&](auto rac) __attribute__((always_inline)) {
    constexpr int RA = decltype(rac)::value;
    {
      const uint8_t* b0 = smem;
#pragma unroll
      for (int r = 0; r < RA; r++) load_x(b0, r, std::integral_constant<int, 0>{});
#pragma unroll
      for (int j = 0; j < (LATE ? CW : CW - 2); j++) load_w(b0, j);
      load_ws(b0, std::integral_constant<int, 0>{});
    }
#pragma unroll
    for (int r = 0; r < RW; r++)
#pragma unroll
      for (int j = 0; j < CW; j++)
#pragma unroll
        for (int i = 0; i < 16; i++) acc[r][j][i] = 0.f;

    // One K step.  Stage kt+1 (my copies landed) becomes everyone's at the barrier; every wave has by
    // then finished all reads of stage kt-1 (they fed the MFMAs of step kt-1), so that slot takes the
    // stage D - 1 steps ahead, if there is one.  Stages kt+2 .. min(kt+D-2, nkt-1) may stay in flight.
    // MAIN steps (kt + D - 1 < nkt) interleave their copies with the MFMAs; the last steps of an item
    // issue any copy up front and wait by a runtime count.
    auto step = [&](int kt, auto pc, auto mc) __attribute__((always_inline)) {
      constexpr int P = decltype(pc)::value;
      constexpr bool MAIN = decltype(mc)::value;
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (!LATE) {
        if constexpr (MAIN)
          wait_vmcnt<C::kOps * (D - 3)>();
        else
          wait_stages(nkt - kt - 2, std::integral_constant<int, D - 3>{});
        block_sync();
        __builtin_amdgcn_sched_barrier(0);
      }
      const int kn = kt + 1 < nkt ? kt + 1 : kt;
      const uint8_t* cb = smem + (kt % D) * C::kStage;
      const uint8_t* nb = smem + (kn % D) * C::kStage;
      const int s = kt + D - 1;
      if constexpr (!MAIN) {
        if (s < nkt) issue(cur, s, s % D);
        __builtin_amdgcn_sched_barrier(0);
      }
      static_for<0, Plan::NM>([&](auto mi) __attribute__((always_inline)) {
        constexpr int m = decltype(mi)::value;
        mfma_one(mi, pc, rac);
        static_for<0, Plan::kCap>([&](auto ci) __attribute__((always_inline)) {
          constexpr int task = plan.t[m][decltype(ci)::value];
          if constexpr (task >= StepTask::kDma) {
            if constexpr (MAIN) issue_op(cur, s, s % D, std::integral_constant<int, task - StepTask::kDma>{});
          } else if constexpr (task >= StepTask::kRel) {
            load_w(nb, task - StepTask::kRel);
          } else if constexpr (task == StepTask::kWs) {
            load_ws(nb, std::integral_constant<int, 1 - P>{});
          } else if constexpr (task >= StepTask::kX) {
            if constexpr (task - StepTask::kX < RA) load_x(nb, task - StepTask::kX, std::integral_constant<int, 1 - P>{});
          } else if constexpr (task >= StepTask::kDef) {
            load_w(cb, CW - 2 + task - StepTask::kDef);
          }
        });
        __builtin_amdgcn_sched_barrier(0);
      });
      if constexpr (LATE) {
        // Stage kt+1 (my copies landed) becomes everyone's at the barrier; the stages after it
        // (kt+2 .. min(kt+D-1, nkt-1), this step's copies among them) may stay in flight.  Every wave
        // has by then finished reading stage kt (its fragments fed this step's MFMAs), so the next
        // step may copy into that slot.
        if (kt + 1 < nkt) {
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (MAIN)
            wait_vmcnt<C::kOps * (D - 2)>();
          else
            wait_stages(nkt - kt - 2, std::integral_constant<int, D - 2>{});
          block_sync();
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int r = 0; r < RA; r++) load_x(nb, r, std::integral_constant<int, 1 - P>{});
#pragma unroll
          for (int j = 0; j < CW; j++) load_w(nb, j);
          load_ws(nb, std::integral_constant<int, 1 - P>{});
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    // main steps in pairs (an even count, so the buffers are back in place), then the rest
    const int nmain = nkt > D - 1 ? ((nkt - (D - 1)) & ~1) : 0;
    int kt = 0;
    for (; kt < nmain; kt += 2) {
      step(kt, std::integral_constant<int, 0>{}, std::true_type{});
      step(kt + 1, std::integral_constant<int, 1>{}, std::true_type{});
    }
    for (; kt + 2 <= nkt; kt += 2) {
      step(kt, std::integral_constant<int, 0>{}, std::false_type{});
      step(kt + 1, std::integral_constant<int, 1>{}, std::false_type{});
    }
    if (kt < nkt) step(kt, std::integral_constant<int, 0>{}, std::false_type{});
    };
    {
      const int nreal = (nrows + 31) >> 5;  // row groups holding pairs
      if constexpr (RW == 2) {
        if (wr + WR < nreal)
          kloop(std::integral_constant<int, 2>{});
        else if (wr < nreal)
          kloop(std::integral_constant<int, 1>{});
        else
          kloop(std::integral_constant<int, 0>{});
      } else {
        if (wr < nreal)
          kloop(std::integral_constant<int, RW>{});
        else
          kloop(std::integral_constant<int, 0>{});
      }
    }

    // ---- next item's first D - 1 stages go out before this item's epilogue, so their latency hides
    // under it.  make_src reads the next item's token table, whose copy went out at this item's start:
    // every copy of this wave is waited for here (the interleaved plan's last step has already waited
    // for all of them, and so has a late-load item of two or more K steps; a late-load item of one K
    // step has not), and the barrier then makes every wave's table copies visible and every wave done
    // reading the ring.
    if (has_next) {
      wait_vmcnt<0>();
      block_sync();
      make_src(item_of(q + 1), tb ^ 1, cur);
#pragma unroll
      for (int s = 0; s < D - 1; s++)
        if (s < nkt) issue(cur, s, s);
    }

    // ---- epilogue (one tile or tile pair at a time: the scheduling barriers keep each one's values
    // short-lived)
    if constexpr (G1) {
#pragma unroll
      for (int r = 0; r < RW; r++) {
        const int rgl = wr + WR * r;
        if (rgl * 32 >= nrows) continue;
#pragma unroll
        for (int p = 0; p < CW / 4; p++) {
          const int it = (x * NT + wc * CW) / 2 + 2 * p;  // even: a K step of the second GEMM
          const int il = (wc * CW) / 2 + 2 * p;           // activation tile within the item
          if (it + 1 < a.ntl)
            g1_epilogue_pair<BIAS, true, AF>(acc[r][4 * p], acc[r][4 * p + 1], acc[r][4 * p + 2], acc[r][4 * p + 3], a,
                                         (lds_u16*)&t_b[tb][0][il * 32], (lds_u16*)&t_b[tb][G1 ? 1 : 0][il * 32],
                                         it >> 1, (prow0 >> 5) + rgl, lane);
          else if (it < a.ntl)
            g1_epilogue_pair<BIAS, false, AF>(acc[r][4 * p], acc[r][4 * p + 1], acc[r][4 * p + 2], acc[r][4 * p + 3], a,
                                          (lds_u16*)&t_b[tb][0][il * 32], (lds_u16*)&t_b[tb][G1 ? 1 : 0][il * 32],
                                          it >> 1, (prow0 >> 5) + rgl, lane);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
      // Lane l holds token row l % 32 of its row group and output columns 8*jj + 4*(l/32) + i of each
      // tile; after one exchange of lane halves, half h holds the 16 consecutive columns 16h .. 16h+15
      // of the row: one block with a power-of-two scale (largest magnitude in [2^13, 2^14) after
      // scaling), converted to 16 integers (round to nearest even) plus the exponent byte: an absolute
      // error of at most 2^-14 of the block maximum.  A second exchange leaves each lane the 64 bytes of
      // one tile of a tile pair, and the pair's 32 rows of 128 bytes go out through this wave's part of
      // ring stage D - 1 (unused until the next item's first step): written one row per lane pair, read
      // back eight lanes per row, so each store instruction writes eight whole 128-byte row segments
      // rather than 32-byte pieces of 32 rows; a pair's read-back completes while the next pair is
      // computed, and its stores follow that (a wave's LDS accesses complete in order, so the next
      // pair's rows may go to the same place).  The exponent bytes of the wave's CW tiles are gathered
      // the same way into CW consecutive bytes per lane.  Rows of a row group past the expert's pairs
      // (padding rows, or the dense layer's rows past M) are not stored.
      const int m = lane & 31, h = lane >> 5;
      const int srow = lane >> 3, sch = lane & 7;  // read-back: row within eight, 16-byte chunk
      constexpr int kStRow = 144;                  // a staged row: 128 bytes + 16 (spreads the banks)
      static_assert(4 * 32 * kStRow <= C::kStage, "the staging rows fit one ring stage");
      typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
      __attribute__((address_space(3))) uint8_t* stg =
          (__attribute__((address_space(3))) uint8_t*)(smem + (D - 1) * C::kStage + wave * (32 * kStRow));
      // without a next item no barrier followed the K loop: another wave may still read stage D - 1
      if (!has_next) block_sync();
      const int ntw0 = x * NT + wc * CW;  // first tile of this wave
      // FULL: every tile of the wave is inside the output (no per-pair checks, so no branches between
      // the pairs and the read-back of one pair stays in flight across the next pair's arithmetic)
      auto epi = [&](auto dc, auto fc) __attribute__((always_inline)) {
        constexpr bool DENSE = decltype(dc)::value, FULL = decltype(fc)::value;
        uint16_t* const obase = DENSE ? a.ydense : a.o16;
#pragma unroll
        for (int r = 0; r < RW; r++) {
          const int rgl = wr + WR * r;
          if (rgl * 32 >= nrows) continue;
          const float wt = __builtin_bit_cast(float, t_row[tb][rgl * 32 + m]);
          const int64_t prow_rg = prow0 + rgl * 32;
          uint32_t eb[2] = {0u, 0u};  // exponent bytes of tiles 0 .. CW/2 - 1 and CW/2 .. CW - 1
          const bool rg_full = rgl * 32 + 32 <= nrows;
          const int glim = rg_full ? 32 : nrows - rgl * 32;  // rows of this group that are stored
          // the staged pair whose stores are pending: its first tile (-1: none) and its read-back
          int pnt = -1;
          u32x4_t sv[4];
          auto store_pending = [&]() __attribute__((always_inline)) {
            if constexpr (FULL) {
              // buffer stores over the group's stored rows: a row past them falls outside the buffer
              // range and is dropped, so no lane mask (and no branch) is needed
              const __amdgpu_buffer_rsrc_t rs =
                  __builtin_amdgcn_make_buffer_rsrc(obase + prow_rg * a.H, (short)0, glim * a.H * 2, kBufFlags);
              const int vo = srow * a.H * 2 + (pnt * 32 + sch * 8) * 2;
#pragma unroll
              for (int s = 0; s < 4; s++) __builtin_amdgcn_raw_buffer_store_b128(sv[s], rs, vo, s * 16 * a.H, 0);
              return;
            }
            // chunks 4 .. 7 are tile pnt + 1, which is past the output when H / 32 is odd; row 8s + srow
            // of the group is 8s rows (8s * H / 8 chunks) past the first
            const bool second = pnt + 1 < a.ntl;
            u32x4_t* op = reinterpret_cast<u32x4_t*>(obase + (prow_rg + srow) * a.H + pnt * 32 + sch * 8);
            if (second && rg_full) {
#pragma unroll
              for (int s = 0; s < 4; s++) op[(int64_t)s * a.H] = sv[s];
            } else {
              const bool col = sch < 4 || second;
              const int lim = nrows - rgl * 32;  // rows of this group that are stored
#pragma unroll
              for (int s = 0; s < 4; s++)
                if (col && 8 * s + srow < lim) op[(int64_t)s * a.H] = sv[s];
            }
          };
#pragma unroll
          for (int jp = 0; jp < CW / 2; jp++) {
            const int nt0 = ntw0 + 2 * jp;
            if (!FULL && nt0 >= a.ntl) continue;
            uint32_t hv[2][8];
#pragma unroll
            for (int t = 0; t < 2; t++) {
              const int j = 2 * jp + t;
              // v[c]: column 16h + c of the tile after the exchange; the tile's 16 values are read
              // first (each read is a scheduling boundary), then exchanged
              float v[16], ra[16];
#pragma unroll
              for (int i = 0; i < 16; i++) ra[i] = acc_read(acc[r][j][i]);
#pragma unroll
              for (int i = 0; i < 4; i++) {
                float x0 = ra[i], x2 = ra[8 + i];
                float x1 = ra[4 + i], x3 = ra[12 + i];
                swap_halves(x0, x2);  // half 0: cols i | 4 + i;  half 1: cols 16 + i | 20 + i
                swap_halves(x1, x3);  // half 0: cols 8 + i | 12 + i;  half 1: cols 24 + i | 28 + i
                v[i] = x0;
                v[4 + i] = x2;
                v[8 + i] = x1;
                v[12 + i] = x3;
              }
              if constexpr (BIAS) {
                lds_u16* bp = (lds_u16*)&t_b[tb][0][(wc * CW + j) * 32 + 16 * h];
                float b[16];
#pragma unroll
                for (int c = 0; c < 4; c++) bias4(bp + 4 * c, b + 4 * c);
#pragma unroll
                for (int c = 0; c < 16; c++) v[c] += b[c];
              }
              if constexpr (DENSE) {
                // dense linear layer (one expert, unit row weights): the row of y itself, bf16
#pragma unroll
                for (int c = 0; c < 8; c++)
                  hv[t][c] = f32_to_bf16_bits(v[2 * c]) | (f32_to_bf16_bits(v[2 * c + 1]) << 16);
              } else {
                // The block maximum of w * v is |w| times that of v (rounding is monotonic), and scaling
                // by a power of two commutes with rounding, so w * 2^-ex is applied as one factor.
                float amax = 0.f;
#pragma unroll
                for (int c = 0; c < 16; c++) amax = fmaxf(amax, fabsf(v[c]));
                amax *= fabsf(wt);
                int ex = amax > 0.f ? __builtin_amdgcn_frexp_expf(amax) - 14 : 0;
                ex = ex < -127 ? -127 : (ex > 127 ? 127 : ex);
                const float f = __builtin_ldexpf(wt, -ex);
                // v * f rounded once to the nearest integer (even on ties): fma(v, f, 1.5 * 2^23) is exact
                // up to that rounding while |v * f| < 2^22 (here < 2^14 + 1), and the sum's low 16 bits are
                // the integer in two's complement; one byte permute packs a pair.
                constexpr float kRound = 12582912.0f;  // 1.5 * 2^23
#pragma unroll
                for (int c = 0; c < 8; c++) {
                  const uint32_t u0 = __float_as_uint(__builtin_fmaf(v[2 * c], f, kRound));
                  const uint32_t u1 = __float_as_uint(__builtin_fmaf(v[2 * c + 1], f, kRound));
                  hv[t][c] = __builtin_amdgcn_perm(u1, u0, 0x05040100u);  // low half of u0, then of u1
                }
                eb[j / (CW / 2)] |= (uint32_t)(ex + 127) << (8 * (j % (CW / 2)));
              }
            }
            // the previous pair's read-back has landed while this pair was computed
            __builtin_amdgcn_sched_barrier(0);
            if (FULL ? jp > 0 : pnt >= 0) store_pending();
            __builtin_amdgcn_sched_barrier(0);
            // half h takes tile nt0 + h whole: hv[0] its columns 0 .. 15, hv[1] columns 16 .. 31
#pragma unroll
            for (int d = 0; d < 8; d++) swap_halves_u32(hv[0][d], hv[1][d]);
            __attribute__((address_space(3))) uint8_t* wrow = stg + m * kStRow + h * 64;
            *(lds_u32x4*)(wrow + 0) = u32x4_t{hv[0][0], hv[0][1], hv[0][2], hv[0][3]};
            *(lds_u32x4*)(wrow + 16) = u32x4_t{hv[0][4], hv[0][5], hv[0][6], hv[0][7]};
            *(lds_u32x4*)(wrow + 32) = u32x4_t{hv[1][0], hv[1][1], hv[1][2], hv[1][3]};
            *(lds_u32x4*)(wrow + 48) = u32x4_t{hv[1][4], hv[1][5], hv[1][6], hv[1][7]};
            // read back: lane chunk sch of row 8s + srow
#pragma unroll
            for (int s = 0; s < 4; s++) sv[s] = *(lds_u32x4*)(stg + (8 * s + srow) * kStRow + sch * 16);
            pnt = nt0;
            __builtin_amdgcn_sched_barrier(0);
          }
          if (pnt >= 0) store_pending();
          if constexpr (!DENSE) {
            // lane (m, h) holds exponent byte j of tile ntw0 + j, columns 16h ..: after one exchange
            // and a byte interleave, lane (m, h) has the CW bytes 2 * ntw0 + CW * h .. of row m
            swap_halves_u32(eb[0], eb[1]);
            const uint32_t lo = __builtin_amdgcn_perm(eb[1], eb[0], 0x05010400u);
            const uint32_t hi = __builtin_amdgcn_perm(eb[1], eb[0], 0x07030602u);
            const int pos = 2 * ntw0 + CW * h;
            uint8_t* sp = a.osc + (prow_rg + m) * (a.H / 16) + pos;
            if (FULL && (a.H / 16) % CW == 0) {
              const __amdgpu_buffer_rsrc_t rs =
                  __builtin_amdgcn_make_buffer_rsrc(a.osc + prow_rg * (a.H / 16), (short)0, glim * (a.H / 16), kBufFlags);
              if constexpr (CW == 8)
                __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{lo, hi}, rs, m * (a.H / 16) + pos, 0, 0);
              else
                __builtin_amdgcn_raw_buffer_store_b32(lo, rs, m * (a.H / 16) + pos, 0, 0);
            } else if (rgl * 32 + m >= nrows) {
            } else if ((FULL || ntw0 + CW <= a.ntl) && (a.H / 16) % CW == 0) {
              if constexpr (CW == 8)
                *reinterpret_cast<u32x2_t*>(sp) = u32x2_t{lo, hi};
              else
                *reinterpret_cast<uint32_t*>(sp) = lo;
            } else {
#pragma unroll
              for (int b = 0; b < CW; b++)
                if (pos + b < 2 * a.ntl) sp[b] = (uint8_t)((b < 4 ? lo : hi) >> (8 * (b & 3)));
            }
          }
        }
      };
      const bool full = ntw0 + CW <= a.ntl;
      if (a.ydense) {
        if (full)
          epi(std::true_type{}, std::true_type{});
        else
          epi(std::true_type{}, std::false_type{});
      } else {
        if (full)
          epi(std::false_type{}, std::true_type{});
        else
          epi(std::false_type{}, std::false_type{});
      }
    }

    if (++q >= nq) break;
    item = item_of(q);
  }
}

template <bool G1, int AF, bool BIAS, int WR, int WC, int RW, int CW, int D>
int launch_cfg(const GemmArgs& a, int64_t max_tiles, hipStream_t stream) {
  constexpr int OCC = Lds<G1, AF, BIAS, WR, WC, RW, CW, D>::kOcc;
  using C = Cfg<G1, AF, WR, WC, RW, CW, D>;
  const int64_t nx = (int64_t)a.ncb * kCB / C::NT;
  int64_t items = max_tiles * nx;
  int64_t grid = 256 * OCC;
  if (items < grid) grid = items;
  grid = kXcds * cdiv(grid, kXcds);
  if (grid < kXcds) grid = kXcds;
  hipLaunchKernelGGL((grouped_gemm_kernel<G1, AF, BIAS, WR, WC, RW, CW, D, OCC>), dim3((unsigned)grid), dim3(256), 0,
                     stream, a);
  return hipGetLastError() == hipSuccess ? MXFP4_OK : MXFP4_ERR_DEVICE;
}

// Tile configurations by rows per M tile (32 * NRG): 1 row group for decode-like loads, 2 or 4 (first
// GEMM only) for larger ones.  The 128-row first GEMM covers a whole column block per workgroup, one
// workgroup per CU; the others run two workgroups per CU where their LDS allows, so that one's stores
// and waits overlap the other's MFMAs.
template <int AF, bool BIAS>
int gemm1_cfg(int NRG, const GemmArgs& a, int64_t max_tiles, hipStream_t stream) {
  switch (NRG) {
    case 1: return launch_cfg<true, AF, BIAS, 1, 4, 1, 4, 3>(a, max_tiles, stream);
    case 2:
      // the three-term operand of the bf16 path needs more registers than two workgroups per CU leave:
      // one workgroup per CU with a 5-stage ring (and interleaved fragment loads)
      if constexpr (AF == kActBf16) return launch_cfg<true, AF, BIAS, 1, 4, 2, 4, 5>(a, max_tiles, stream);
      else return launch_cfg<true, AF, BIAS, 1, 4, 2, 4, 3>(a, max_tiles, stream);
    case 4: return launch_cfg<true, AF, BIAS, 2, 2, 2, 8, 4>(a, max_tiles, stream);
    default: return MXFP4_ERR_SHAPE;
  }
}

template <int AF, bool BIAS>
int gemm2_cfg(int NRG, const GemmArgs& a, int64_t max_tiles, hipStream_t stream) {
  switch (NRG) {
    case 1: return launch_cfg<false, AF, BIAS, 1, 4, 1, 4, 3>(a, max_tiles, stream);
    case 2:
      // the bf16 path's second GEMM runs 32- or 128-row tiles (the placement's tile list follows it)
      if constexpr (AF == kActBf16) return MXFP4_ERR_SHAPE;
      else return launch_cfg<false, AF, BIAS, 1, 4, 2, 4, 3>(a, max_tiles, stream);
    case 4:
      // the first GEMM's 128-row shape (one workgroup per CU, interleaved fragment loads)
      if constexpr (AF == kActBf16) return launch_cfg<false, AF, BIAS, 2, 2, 2, 8, 4>(a, max_tiles, stream);
      else return MXFP4_ERR_SHAPE;
    default: return MXFP4_ERR_SHAPE;
  }
}

template <int AF>
int gemm1_launch(int NRG, const GemmArgs& a, int64_t max_tiles, hipStream_t stream) {
  return a.bias ? gemm1_cfg<AF, true>(NRG, a, max_tiles, stream) : gemm1_cfg<AF, false>(NRG, a, max_tiles, stream);
}

template <int AF>
int gemm2_launch(int NRG, const GemmArgs& a, int64_t max_tiles, hipStream_t stream) {
  return a.bias ? gemm2_cfg<AF, true>(NRG, a, max_tiles, stream) : gemm2_cfg<AF, false>(NRG, a, max_tiles, stream);
}

}  // namespace
