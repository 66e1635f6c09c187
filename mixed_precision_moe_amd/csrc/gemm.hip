// Grouped expert GEMMs of the MoE layer on gfx950 block-scaled MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4), with the SwiGLU and the routing-weighted output fused into
// their epilogues, and the final combine over the top-k experts of each token.
//
// [NS: grouped w13 GEMM, SwiGLU = silu(w1 half) * (w3 half), grouped w2 GEMM, weighted top-k combine;
//  MXFP4 weights with E8M0 scales per 32 elements; P1 Implementation breakdown: the mixed-input fused
//  MoE multiplies packed 4-bit weights with per-32 group scales by 16-bit activations]
//
// The MFMA has no bf16 operand, so a bf16 activation enters as two E2M3 (FP6) terms x = t0 + t1, each
// with its own E8M0 scale per 32 elements, and every product is issued once per term against the same
// FP4 weight registers; FP6 x FP4 runs at the FP4 rate on gfx950.  The first GEMM's output (the SwiGLU
// activation) stays fp32 until it is split into the second GEMM's two terms, and the second GEMM's rows
// are block-scaled fp16 that the combine sums in fp32, so the only bf16 rounding after the input is the
// output's.
//
// First GEMM, transposed: D[n][m] = sum_k W13[n][k] x[m][k], weights as the A operand (rows n = 32
// gate or up rows of one tile), tokens as the B operand (columns m = 32 tokens gathered through the
// padded row order).  Lane l of the 32x32 result holds token l%32 and rows 8*jj + 4*(l/32) + i, so
// gate and up of one column sit in the same lane (SwiGLU in registers) and a 32-element block of the
// activation is split over the two lane halves (one exchange for the block maximum).
//
// Second GEMM, not transposed: D[m][n] = sum_k act[m][k] W2[n][k]; lane l holds output column l%32 and
// rows 8*jj + 4*(l/32) + i.  Its rows go to o16 (fp16 with a power-of-two exponent per 16 rows of a
// column, which keeps about eleven significant bits of every value that matters for the sum) in the
// padded row order; the combine gathers each token's k rows.
//
// Both GEMMs run one kernel template.  A workgroup of four waves (WR x WC) computes an M tile of
// NRG = WR*RW row groups of 32 rows against NT = WC*CW weight tiles of 32 columns; wave (wr, wc) holds
// RW x CW accumulators.  Per 64-wide K step the workgroup copies the step's operands global -> LDS
// with LDS DMA (global_load_lds: no registers, no address math beyond the source) into a ring of D
// stages: every wave issues the same number of copies per stage, waits for its own with vmcnt and one
// barrier per step publishes the stage.  Operand fragments of step kt+1 are read from LDS while the
// MFMAs of step kt run.  Work items (M tile, column position) are dealt to XCDs in contiguous ranges
// so the column positions of one M tile (same gathered tokens) and consecutive tiles of one expert
// (same weights) share an XCD's L2.
#include <type_traits>

#include "common.h"

namespace {

typedef decltype(__builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(bf16x32_t{}, 1.0f)) fp6x32_t;
typedef __attribute__((address_space(3))) void* lds_vptr_t;

constexpr int kFp4 = 4, kFp6 = 2;  // MFMA operand format codes (E2M1, E2M3)
constexpr int kXcds = 8;           // workgroup b runs on XCD b % 8

MX_DEV u32x4_t ld16(const uint8_t* p) { return *reinterpret_cast<const u32x4_t*>(p); }
MX_DEV u32x2_t ld8(const uint8_t* p) { return *reinterpret_cast<const u32x2_t*>(p); }

// LDS DMA: lane i copies 16 (or 4) bytes from its global address to lds_wave_base + i * 16 (or 4).
// (Sub-dword copies still occupy a dword per lane in LDS, so every copied record here is a dword or
// a multiple of 16 bytes.)
MX_DEV void dma16(const void* g, uint8_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_vptr_t)lds_wave_base, 16, 0, 0);
}
MX_DEV void dma4(const void* g, uint8_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_vptr_t)lds_wave_base, 4, 0, 0);
}

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

// ------------------------------------------------------------------------------------------------
// Kernel configuration.  LDS stage: [NT weight pieces of 1 KB][1 KB weight scale records of the
// column block][NRG x 3 KB activation slots, lane-major][NRG x 256 B activation scale dwords].
template <int WR, int WC, int RW, int CW, int D>
struct Cfg {
  static constexpr int NRG = WR * RW, NT = WC * CW;
  static_assert(WR * WC == 4, "four waves");
  static_assert(NT == 8 || NT == 16, "a workgroup covers a column block or half of one");
  static_assert(CW % 4 == 0, "weight scales are read four tiles per dword");
  static_assert(D >= 3 && D <= 6, "ring depth");  // stages issued D - 1 steps ahead
  static constexpr int oW = 0, oWS = NT * 1024, oX = oWS + 1024, oXS = oX + NRG * 3072;
  static constexpr int kStage = oXS + NRG * 256;
  static constexpr int nW = NT / 4;              // weight pieces copied per wave
  static constexpr int nX = (3 * NRG + 3) / 4;   // 1 KB activation copies per wave (last one repeated)
  static constexpr int nXS = (NRG + 3) / 4;      // activation scale copies per wave
  static constexpr int kOps = nW + 1 + nX + nXS; // copies per wave per stage
};


// First GEMM epilogue for one (32-column activation tile `it`, row group `rg`) result held by one
// wave: bias, SwiGLU in fp32, then the two-term E2M3 split of each 32-element block (one block = the
// two lane halves of a token column; each block maximum needs one exchange across the halves), written
// in the second GEMM's operand layout.  The last K step of the second GEMM is completed with a zero
// block when I/32 is odd.
MX_DEV void g1_epilogue_tile(const f32x16_t& accg, const f32x16_t& accu, const GemmArgs& a, int e, int it, int rg,
                             int lane) {
  const uint16_t* __restrict__ b13 = a.bias;
  const int m = lane & 31, h = lane >> 5;
  float cur[16];
#pragma unroll
  for (int jj = 0; jj < 4; jj++) {
    // accumulator 4*jj + i holds row 8*jj + 4*h + i of the tile: four consecutive bias entries
    float b1[4] = {0.f, 0.f, 0.f, 0.f}, b3[4] = {0.f, 0.f, 0.f, 0.f};
    if (b13) {
      const uint16_t* bp = b13 + (int64_t)e * 2 * a.I + it * 32 + 8 * jj + 4 * h;
      const u32x2_t v1 = *reinterpret_cast<const u32x2_t*>(bp);
      const u32x2_t v3 = *reinterpret_cast<const u32x2_t*>(bp + a.I);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        b1[i] = bf16_bits_to_f32((v1[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
        b3[i] = bf16_bits_to_f32((v3[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float gt = accg[4 * jj + i] + b1[i];
      // silu(g) = g / (1 + exp(-g)) with the hardware exponential and reciprocal (exp overflow gives 0)
      cur[4 * jj + i] = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * (accu[4 * jj + i] + b3[i]);
    }
  }
  const int kt2 = it >> 1, kb = it & 1;
  const int slot = (rg * a.nkt2 + kt2) * 64 + kb * 32 + m;
  uint32_t* chunk = reinterpret_cast<uint32_t*>(a.actq + (int64_t)slot * kSlot + h * 12);
  uint32_t scales = 0;
  // Each term quantizes the bf16 rounding of the fp32 remainder (the remainder itself stays fp32).
  // Rounding is monotonic, so the largest bf16 magnitude is the rounding of the largest fp32 one.
#pragma unroll
  for (int term = 0; term < kTerms; term++) {
    float amax = 0.f;
    bf16x32_t v;
#pragma unroll
    for (int q = 0; q < 16; q += 2) {
      amax = fmaxf(amax, fmaxf(fabsf(cur[q]), fabsf(cur[q + 1])));
      const bf16x2_t two = __builtin_convertvector((f32x2_t){cur[q], cur[q + 1]}, bf16x2_t);
      v[q] = two[0];
      v[q + 1] = two[1];
      v[16 + q] = __builtin_bit_cast(__bf16, (uint16_t)0);
      v[17 + q] = __builtin_bit_cast(__bf16, (uint16_t)0);
    }
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    const bf16x2_t am = __builtin_convertvector((f32x2_t){amax, 0.f}, bf16x2_t);
    const uint32_t ex = e8m0_from_amax_bits((uint32_t)__builtin_bit_cast(uint16_t, am[0]) << 16);
    const float sv = e8m0_as_scale_operand(ex);
    const fp6x32_t codes = __builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(v, sv);
    chunk[term * 6] = codes[0];
    chunk[term * 6 + 1] = codes[1];
    chunk[term * 6 + 2] = codes[2];
    scales |= ex << (8 * term);
    if (term + 1 < kTerms) {
      const auto deq = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(codes, sv);
#pragma unroll
      for (int q = 0; q < 16; q++) cur[q] = cur[q] - deq[q];
    }
  }
  if (h == 0) reinterpret_cast<uint32_t*>(a.acts)[slot] = scales;
  if ((it == a.ntl - 1) && (a.ntl & 1)) {
    const int zslot = (rg * a.nkt2 + kt2) * 64 + 32 + m;
    uint32_t* zp = reinterpret_cast<uint32_t*>(a.actq + (int64_t)zslot * kSlot + h * (kSlot / 2));
#pragma unroll
    for (int q = 0; q < kSlot / 8; q++) zp[q] = 0;
    if (h == 0) reinterpret_cast<uint32_t*>(a.acts)[zslot] = 0;
  }
}

// ------------------------------------------------------------------------------------------------
// The grouped GEMM.  G1: first GEMM (A = weights, B = gathered token terms, SwiGLU epilogue);
// otherwise the second GEMM (A = activation terms, B = weights, weighted fp32 rows to o_buf).
template <bool G1, int WR, int WC, int RW, int CW, int D, int OCC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(OCC))) void grouped_gemm_kernel(GemmArgs a) {
  using C = Cfg<WR, WC, RW, CW, D>;
  constexpr int NRG = C::NRG, NT = C::NT;
  __shared__ __attribute__((aligned(16))) uint8_t smem[D * C::kStage];
  const int tid = threadIdx.x;
  const int nkt = a.nkt, ncb = a.ncb;
  const int nx = ncb * kCB / NT;
  const int nblk = a.nblk;  // token slots per row of xq (first GEMM)

  const int total = *a.ntiles * nx;
  const int chunk = (total + kXcds - 1) / kXcds;
  const int xcd = blockIdx.x % kXcds, per_xcd = gridDim.x / kXcds;

  for (int p = blockIdx.x / kXcds; p < chunk; p += per_xcd) {
    const int item = xcd * chunk + p;
    if (item >= total) break;
    // Lane and wave indices are re-derived per item through volatile asm so that nothing computed from
    // them is hoisted out of the item loop and kept live across the K loop.
    int lane, wave;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
    asm volatile("s_lshr_b32 %0, %1, 6" : "=s"(wave) : "s"(__builtin_amdgcn_readfirstlane(tid)));
    const int wr = wave / WC, wc = wave % WC;
    const int tile = item / nx, x = item % nx;
    const int4 td = a.tiles[tile];
    const int e = td.x, prow0 = td.y, nrows = td.z;
    const int cb = x * NT / kCB;
    const int jj0 = (x * NT) % kCB;

    // ---- copy sources of this item (step 0; each stage advances by a fixed stride)
    const int64_t wstep0 = (int64_t)(e * ncb + cb) * nkt;  // first K step of this (expert, column block)
    const uint8_t* wsrc = a.wq + wstep0 * (kCB * 1024) + (jj0 + wave * C::nW) * 1024 + lane * 16;
    const uint8_t* wssrc = a.ws + wstep0 * 1024 + wave * 256 + lane * 4;
    const uint8_t* xsrc[C::nX];
    int xdst[C::nX];
#pragma unroll
    for (int q = 0; q < C::nX; q++) {
      int o = wave + 4 * q;
      o = o < 3 * NRG ? o : 3 * NRG - 1;
      const int rg = o / 3, pp = o % 3;
      xdst[q] = C::oX + o * 1024;
      if (G1) {
        const int c = pp * 64 + lane, s = c / 3, part = c % 3;
        const int tok = a.prow_tok[prow0 + rg * 32 + (s & 31)];
        xsrc[q] = a.xq + ((int64_t)tok * nblk + (s >> 5)) * kSlot + part * 16;
      } else {
        xsrc[q] = a.xq + (int64_t)((prow0 >> 5) + rg) * nkt * (64 * kSlot) + (pp * 64 + lane) * 16;
      }
    }
    const uint8_t* xssrc[C::nXS];
    int xsdst[C::nXS];
#pragma unroll
    for (int q = 0; q < C::nXS; q++) {
      int o = wave + 4 * q;
      o = o < NRG ? o : NRG - 1;
      xsdst[q] = C::oXS + o * 256;
      if (G1) {
        const int tok = a.prow_tok[prow0 + o * 32 + (lane & 31)];
        xssrc[q] = a.xs + ((int64_t)tok * nblk + (lane >> 5)) * 4;
      } else {
        xssrc[q] = a.xs + (int64_t)((prow0 >> 5) + o) * nkt * 256 + lane * 4;
      }
    }
    constexpr int xstep = G1 ? 2 * kSlot : 64 * kSlot;  // bytes per K step of an activation copy
    constexpr int xsstep = G1 ? 8 : 256;

    auto issue = [&](int s, int slot) __attribute__((always_inline)) {
      const int kt = s < nkt ? s : nkt - 1;  // past the end: repeat the last stage (never read)
      uint8_t* base = smem + slot * C::kStage;
#pragma unroll
      for (int i = 0; i < C::nW; i++) dma16(wsrc + kt * (kCB * 1024) + i * 1024, base + C::oW + (wave * C::nW + i) * 1024);
      dma4(wssrc + kt * 1024, base + C::oWS + wave * 256);
#pragma unroll
      for (int q = 0; q < C::nX; q++) dma16(xsrc[q] + kt * xstep, base + xdst[q]);
#pragma unroll
      for (int q = 0; q < C::nXS; q++) dma4(xssrc[q] + kt * xsstep, base + xsdst[q]);
    };

    wait_vmcnt<0>();  // nothing of the previous item in flight
    block_sync();     // every wave is done with the ring
#pragma unroll
    for (int s = 0; s < D - 1; s++) issue(s, s);

    // Each E2M3 term operand (6 dwords) is read by its own two LDS loads (16 + 8 bytes for term 0 at
    // slot offset 0, 8 + 16 bytes for term 1 at offset 24), so every MFMA operand tuple is written in
    // place by its loads.  Activation fragments are double-buffered across steps; a weight fragment is
    // reloaded for the next step right after the last MFMA that uses it.
    // xop[P]: activation operands (two buffers selected by a compile-time parity), w/wsc: weights.
    i32x8_t xop[2][RW][kTerms];
    uint32_t xsc[2][RW];
    u32x4_t w[CW];
    uint32_t wsc[CW / 4];
    auto load_x = [&](const uint8_t* base, auto pc) __attribute__((always_inline)) {
      constexpr int P = decltype(pc)::value;
#pragma unroll
      for (int r = 0; r < RW; r++) {
        const uint8_t* xp = base + C::oX + (wr * RW + r) * 3072 + lane * kSlot;
        const u32x4_t a4 = ld16(xp);
        const u32x2_t a2 = ld8(xp + 16);
        const u32x2_t b2 = ld8(xp + 24);
        const u32x4_t b4 = ld16(xp + 32);
        xop[P][r][0] = i32x8_t{(int)a4[0], (int)a4[1], (int)a4[2], (int)a4[3], (int)a2[0], (int)a2[1], 0, 0};
        xop[P][r][1] = i32x8_t{(int)b2[0], (int)b2[1], (int)b4[0], (int)b4[1], (int)b4[2], (int)b4[3], 0, 0};
        xsc[P][r] = *reinterpret_cast<const uint32_t*>(base + C::oXS + (wr * RW + r) * 256 + lane * 4);
      }
    };
    auto load_w = [&](const uint8_t* base, int j) __attribute__((always_inline)) { w[j] = ld16(base + C::oW + (wc * CW + j) * 1024 + lane * 16); };
    auto load_ws = [&](const uint8_t* base, int j4) __attribute__((always_inline)) {
      wsc[j4] = *reinterpret_cast<const uint32_t*>(base + C::oWS + lane * 16 + jj0 + wc * CW + j4 * 4);
    };

    f32x16_t acc[RW][CW];
#pragma unroll
    for (int r = 0; r < RW; r++)
#pragma unroll
      for (int j = 0; j < CW; j++)
#pragma unroll
        for (int i = 0; i < 16; i++) acc[r][j][i] = 0.f;

    // MFMAs of weight tiles [J0, J0 + JG): term-major, then row group, then tile, so an accumulator is
    // reused RW * JG instructions later.
    constexpr int JG = 2;
    auto mfma_group = [&](auto jc, auto pc) __attribute__((always_inline)) {
      constexpr int J0 = decltype(jc)::value * JG;
      constexpr int P = decltype(pc)::value;
      static_for<0, kTerms>([&](auto tc) __attribute__((always_inline)) {
        constexpr int t = decltype(tc)::value;
#pragma unroll
        for (int r = 0; r < RW; r++) {
          const i32x8_t xo = xop[P][r][t];
          static_for<J0, J0 + JG>([&](auto jc2) __attribute__((always_inline)) {
            constexpr int j = decltype(jc2)::value;
            const i32x8_t wo = i32x8_t{(int)w[j][0], (int)w[j][1], (int)w[j][2], (int)w[j][3], 0, 0, 0, 0};
            if constexpr (G1)
              acc[r][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wo, xo, acc[r][j], kFp4, kFp6, j & 3,
                                                                          wsc[j >> 2], t, xsc[P][r]);
            else
              acc[r][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(xo, wo, acc[r][j], kFp6, kFp4, t, xsc[P][r],
                                                                          j & 3, wsc[j >> 2]);
          });
        }
      });
    };

    // One K step.  Stage kt+1 (my copies landed) becomes everyone's at the barrier; every wave has by
    // then finished all reads of stage kt-1 (they fed the MFMAs of step kt-1), so that slot takes stage
    // kt + D - 1.  The activation fragments of step kt+1 are read into `xn` at the start, the weight
    // fragments of step kt+1 after their last use in this step.
    auto step = [&](int kt, auto pc) __attribute__((always_inline)) {
      constexpr int P = decltype(pc)::value;
      wait_vmcnt<C::kOps * (D - 3)>();
      block_sync();
      const int kn = kt + 1 < nkt ? kt + 1 : kt;
      const uint8_t* nb = smem + (kn % D) * C::kStage;
      load_x(nb, std::integral_constant<int, 1 - P>{});
      issue(kt + D - 1, (kt + D - 1) % D);
      static_for<0, CW / JG>([&](auto gc) __attribute__((always_inline)) {
        constexpr int J0 = decltype(gc)::value * JG;
        mfma_group(gc, pc);
#pragma unroll
        for (int j = J0; j < J0 + JG; j++) load_w(nb, j);
        if constexpr ((J0 + JG) % 4 == 0) load_ws(nb, (J0 + JG) / 4 - 1);
      });
    };

    // stage 0 visible: D - 2 later stages may still be in flight
    wait_vmcnt<C::kOps * (D - 2)>();
    block_sync();
    {
      const uint8_t* b0 = smem;
      load_x(b0, std::integral_constant<int, 0>{});
#pragma unroll
      for (int j = 0; j < CW; j++) load_w(b0, j);
#pragma unroll
      for (int j4 = 0; j4 < CW / 4; j4++) load_ws(b0, j4);
    }
    int kt = 0;
    for (; kt + 2 <= nkt; kt += 2) {  // two steps per iteration keep both buffers in place
      step(kt, std::integral_constant<int, 0>{});
      step(kt + 1, std::integral_constant<int, 1>{});
    }
    if (kt < nkt) step(kt, std::integral_constant<int, 0>{});

    // ---- epilogue (one tile at a time: the scheduling barriers keep each tile's values short-lived)
    if constexpr (G1) {
#pragma unroll
      for (int r = 0; r < RW; r++) {
        const int rgl = wr * RW + r;
        if (rgl * 32 >= nrows) continue;
#pragma unroll
        for (int i = 0; i < CW / 2; i++) {
          const int it = (x * NT + wc * CW) / 2 + i;
          if (it < a.ntl) g1_epilogue_tile(acc[r][2 * i], acc[r][2 * i + 1], a, e, it, (prow0 >> 5) + rgl, lane);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
      // Rows 8*jj + 4*h + i (h = lane / 32) of each row group, column lane % 32 of each tile: the lane's
      // 16 values of one tile form one block with a power-of-two scale (largest magnitude in
      // [2^14, 2^15) after scaling), stored as fp16 plus the exponent byte.
      const int h = lane >> 5;
#pragma unroll
      for (int r = 0; r < RW; r++) {
        const int rgl = wr * RW + r;
        if (rgl * 32 >= nrows) continue;
        float wt[16];
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
          const f32x4_t w4 = *reinterpret_cast<const f32x4_t*>(a.prow_w + prow0 + rgl * 32 + 8 * jj + 4 * h);
#pragma unroll
          for (int i = 0; i < 4; i++) wt[4 * jj + i] = rgl * 32 + 8 * jj + 4 * h + i < nrows ? w4[i] : 0.f;
        }
        uint16_t* orow = a.o16 + (int64_t)(prow0 + rgl * 32 + 4 * h) * a.H;
        uint8_t* srow = a.osc + (int64_t)(((prow0 >> 5) + rgl) * 2 + h) * a.H;
#pragma unroll
        for (int j = 0; j < CW; j++) {
          const int nt = x * NT + wc * CW + j;
          if (nt < a.ntl) {
            const int col = nt * 32 + (lane & 31);
            const float bb = a.bias ? bf16_bits_to_f32(a.bias[(int64_t)e * a.H + col]) : 0.f;
            float v[16];
            float amax = 0.f;
#pragma unroll
            for (int q = 0; q < 16; q++) {
              v[q] = wt[q] * (acc[r][j][q] + bb);
              amax = fmaxf(amax, fabsf(v[q]));
            }
            int ex = amax > 0.f ? __builtin_amdgcn_frexp_expf(amax) - 15 : 0;
            ex = ex < -127 ? -127 : (ex > 127 ? 127 : ex);
#pragma unroll
            for (int q = 0; q < 16; q++) {
              const int row = rgl * 32 + 8 * (q >> 2) + 4 * h + (q & 3);
              const _Float16 hv = (_Float16)__builtin_ldexpf(v[q], -ex);
              if (row < nrows) orow[(8 * (q >> 2) + (q & 3)) * a.H + col] = __builtin_bit_cast(uint16_t, hv);
            }
            srow[col] = (uint8_t)(ex + 127);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }
}

// y[t] = sum over the token's k pairs of the fp16 rows (times their block powers of two), fp32 sum in
// slot order, bf16 output.  One thread per 8 output columns of a token.
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ o16, const uint8_t* __restrict__ osc,
                                                      const int32_t* __restrict__ pair_prow, uint16_t* __restrict__ y,
                                                      int64_t H, int k, int64_t n) {
  const int64_t H8 = H / 8;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / H8, c = (i - t * H8) * 8;
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; j++) {
      const int64_t r = pair_prow[t * k + j];
      const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(o16 + r * H + c));
      const u32x2_t e = *reinterpret_cast<const u32x2_t*>(osc + (((r >> 5) * 2 + ((r >> 2) & 1)) * H + c));
#pragma unroll
      for (int q = 0; q < 8; q++) {
        const uint16_t hb = (uint16_t)(v[q >> 1] >> (16 * (q & 1)));
        const int ex = (int)((e[q >> 2] >> (8 * (q & 3))) & 0xFFu) - 127;
        s[q] += __builtin_ldexpf((float)__builtin_bit_cast(_Float16, hb), ex);
      }
    }
    u32x4_t o;
#pragma unroll
    for (int q = 0; q < 4; q++) o[q] = f32_to_bf16_bits(s[2 * q]) | (f32_to_bf16_bits(s[2 * q + 1]) << 16);
    reinterpret_cast<u32x4_t*>(y)[i] = o;
  }
}

template <bool G1, int WR, int WC, int RW, int CW, int D, int OCC>
int launch_cfg(const GemmArgs& a, int64_t max_tiles, hipStream_t stream) {
  const int wg_per_cu = OCC;
  using C = Cfg<WR, WC, RW, CW, D>;
  const int64_t nx = (int64_t)a.ncb * kCB / C::NT;
  int64_t items = max_tiles * nx;
  int64_t grid = 256 * wg_per_cu;
  if (items < grid) grid = items;
  grid = kXcds * cdiv(grid, kXcds);
  if (grid < kXcds) grid = kXcds;
  hipLaunchKernelGGL((grouped_gemm_kernel<G1, WR, WC, RW, CW, D, OCC>), dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError() == hipSuccess ? MXFP4_OK : MXFP4_ERR_DEVICE;
}

}  // namespace

// Tile configurations by rows per M tile (32 * NRG): 1 row group for decode-like loads, 2 or 4 for
// larger ones.  The first GEMM covers a whole column block per workgroup; the 128-row second GEMM
// covers half of one so that two workgroups share a CU and one's output stores overlap the other's
// MFMAs.
int launch_gemm1(int NRG, const GemmArgs& a, int64_t max_tiles, hipStream_t stream) {
  switch (NRG) {
    case 1: return launch_cfg<true, 1, 4, 1, 4, 3, 2>(a, max_tiles, stream);
    case 2: return launch_cfg<true, 1, 4, 2, 4, 3, 2>(a, max_tiles, stream);
    case 4: return launch_cfg<true, 2, 2, 2, 8, 5, 1>(a, max_tiles, stream);
    default: return MXFP4_ERR_SHAPE;
  }
}

int launch_gemm2(int NRG, const GemmArgs& a, int64_t max_tiles, hipStream_t stream) {
  switch (NRG) {
    case 1: return launch_cfg<false, 1, 4, 1, 4, 3, 2>(a, max_tiles, stream);
    case 2: return launch_cfg<false, 1, 4, 2, 4, 3, 2>(a, max_tiles, stream);
    case 4: return launch_cfg<false, 2, 2, 2, 4, 3, 2>(a, max_tiles, stream);
    default: return MXFP4_ERR_SHAPE;
  }
}

int launch_combine(const uint16_t* o16, const uint8_t* osc, const int32_t* pair_prow, void* y, int64_t T, int64_t H, int k,
                   hipStream_t stream) {
  const int64_t n = T * (H / 8);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (n > 0)
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, o16, osc, pair_prow, (uint16_t*)y, H,
                       k, n);
  return hipGetLastError() == hipSuccess ? MXFP4_OK : MXFP4_ERR_DEVICE;
}
