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
// activation) stays fp32 until it is split into the second GEMM's two terms, and the second GEMM writes
// fp32 rows that the combine sums in fp32, so the only bf16 rounding after the input is the output's.
//
// First GEMM, transposed: D[n][m] = sum_k W13[n][k] x[m][k], weights as the A operand (rows n = 32
// gate or up rows of one tile), tokens as the B operand (columns m = 32 tokens gathered through the
// padded row order).  Lane l of the 32x32 result holds token l%32 and rows 8*jj + 4*(l/32) + i, so
// gate and up of one column sit in the same lane (SwiGLU in registers) and a 32-element block of the
// activation is split over the two lane halves (one exchange for the block maximum).
//
// Second GEMM, not transposed: D[m][n] = sum_k act[m][k] W2[n][k]; lane l holds output column l%32 and
// rows 8*jj + 4*(l/32) + i, so each store instruction writes 2 x 32 consecutive floats of o_buf.
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

MX_DEV float silu(float g) { return g / (1.0f + __expf(-g)); }

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
MX_DEV void g1_epilogue_tile(const f32x16_t& accg, const f32x16_t& accu, const uint16_t* __restrict__ b13,
                             uint8_t* __restrict__ actq, uint8_t* __restrict__ acts, const MoeGeom& g, int e, int64_t it,
                             int64_t rg, int lane) {
  const int m = lane & 31, h = lane >> 5;
  float cur[16];
#pragma unroll
  for (int q = 0; q < 16; q++) {
    const int n = 8 * (q >> 2) + 4 * h + (q & 3);
    float b1 = 0.f, b3 = 0.f;
    if (b13) {
      b1 = bf16_bits_to_f32(b13[(int64_t)e * 2 * g.I + it * 32 + n]);
      b3 = bf16_bits_to_f32(b13[(int64_t)e * 2 * g.I + g.I + it * 32 + n]);
    }
    cur[q] = silu(accg[q] + b1) * (accu[q] + b3);
  }
  const int64_t kt2 = it >> 1, kb = it & 1;
  const int64_t slot = (rg * g.nkt2 + kt2) * 64 + kb * 32 + m;
  uint8_t* chunk = actq + slot * kSlot;
  uint32_t scales = 0;
  // Each term quantizes the bf16 rounding of the fp32 remainder; the remainder itself stays fp32.
#pragma unroll
  for (int term = 0; term < kTerms; term++) {
    uint32_t rb[16];
    uint32_t amax = 0;
#pragma unroll
    for (int q = 0; q < 16; q++) {
      rb[q] = f32_to_bf16_bits(cur[q]);
      amax = max(amax, rb[q] & 0x7FFFu);
    }
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 32));
    const uint32_t ex = e8m0_from_amax_bits(amax << 16);
    const float sv = e8m0_as_scale_operand(ex);
    bf16x32_t v;
#pragma unroll
    for (int q = 0; q < 16; q++) {
      v[q] = __builtin_bit_cast(__bf16, (uint16_t)rb[q]);
      v[16 + q] = __builtin_bit_cast(__bf16, (uint16_t)0);
    }
    const fp6x32_t codes = __builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(v, sv);
    uint32_t* tp = reinterpret_cast<uint32_t*>(chunk + term * 24 + h * 12);
    tp[0] = codes[0];
    tp[1] = codes[1];
    tp[2] = codes[2];
    scales |= ex << (8 * term);
    if (term + 1 < kTerms) {
      const auto deq = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(codes, sv);
#pragma unroll
      for (int q = 0; q < 16; q++) cur[q] = cur[q] - deq[q];
    }
  }
  if (h == 0) reinterpret_cast<uint32_t*>(acts)[slot] = scales;
  if ((it == g.nit - 1) && (g.nit & 1)) {
    const int64_t zslot = (rg * g.nkt2 + kt2) * 64 + 32 + m;
    uint32_t* zp = reinterpret_cast<uint32_t*>(actq + zslot * kSlot + h * (kSlot / 2));
#pragma unroll
    for (int q = 0; q < kSlot / 8; q++) zp[q] = 0;
    if (h == 0) reinterpret_cast<uint32_t*>(acts)[zslot] = 0;
  }
}

// ------------------------------------------------------------------------------------------------
// The grouped GEMM.  G1: first GEMM (A = weights, B = gathered token terms, SwiGLU epilogue);
// otherwise the second GEMM (A = activation terms, B = weights, weighted fp32 rows to o_buf).
template <bool G1, int WR, int WC, int RW, int CW, int D>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(GemmArgs a) {
  using C = Cfg<WR, WC, RW, CW, D>;
  constexpr int NRG = C::NRG, NT = C::NT;
  __shared__ __attribute__((aligned(16))) uint8_t smem[D * C::kStage];
  const MoeGeom& g = a.g;
  const int tid = threadIdx.x;
  const int64_t nkt = G1 ? g.nkt1 : g.nkt2;
  const int64_t ncb = G1 ? g.ncb1 : g.ncb2;
  const int nx = (int)(ncb * kCB / NT);
  const int64_t nblk = 2 * g.nkt1;  // token slots per row of xq (first GEMM)

  const int64_t total = (int64_t)(*a.ntiles) * nx;
  const int64_t chunk = (total + kXcds - 1) / kXcds;
  const int64_t xcd = blockIdx.x % kXcds, per_xcd = gridDim.x / kXcds;

  for (int64_t p = blockIdx.x / kXcds; p < chunk; p += per_xcd) {
    const int64_t item = xcd * chunk + p;
    if (item >= total) break;
    // Lane and wave indices are re-derived per item through volatile asm so that nothing computed from
    // them is hoisted out of the item loop and kept live across the K loop.
    int lane, wave;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
    asm volatile("s_lshr_b32 %0, %1, 6" : "=s"(wave) : "s"(__builtin_amdgcn_readfirstlane(tid)));
    const int wr = wave / WC, wc = wave % WC;
    const int tile = (int)(item / nx), x = (int)(item % nx);
    const int4 td = a.tiles[tile];
    const int e = td.x, prow0 = td.y, nrows = td.z;
    const int64_t cb = (int64_t)x * NT / kCB;
    const int jj0 = (x * NT) % kCB;

    // ---- copy sources of this item (step 0; each stage advances by a fixed stride)
    const uint8_t* wsrc = a.wq + ((e * ncb + cb) * nkt) * (kCB * 1024) + (jj0 + wave * C::nW) * 1024 + lane * 16;
    const uint8_t* wssrc = a.ws + ((e * ncb + cb) * nkt) * 1024 + wave * 256 + lane * 4;
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
        xsrc[q] = a.xq + (((int64_t)(prow0 >> 5) + rg) * nkt * 64) * kSlot + (pp * 64 + lane) * 16;
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
        xssrc[q] = a.xs + ((((int64_t)(prow0 >> 5) + o) * nkt) * 64 + lane) * 4;
      }
    }
    const int64_t xstep = G1 ? 2 * kSlot : 64 * kSlot;  // bytes per K step of an activation copy
    const int64_t xsstep = G1 ? 8 : 256;

    auto issue = [&](int64_t s, int slot) __attribute__((always_inline)) {
      const int64_t kt = s < nkt ? s : nkt - 1;  // past the end: repeat the last stage (never read)
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
    auto step = [&](int64_t kt, auto pc) __attribute__((always_inline)) {
      constexpr int P = decltype(pc)::value;
      wait_vmcnt<C::kOps * (D - 3)>();
      block_sync();
      const int64_t kn = kt + 1 < nkt ? kt + 1 : kt;
      const uint8_t* nb = smem + (kn % D) * C::kStage;
      load_x(nb, std::integral_constant<int, 1 - P>{});
      issue(kt + D - 1, (int)((kt + D - 1) % D));
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
    int64_t kt = 0;
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
          const int64_t it = ((int64_t)x * NT + wc * CW) / 2 + i;
          if (it < g.nit)
            g1_epilogue_tile(acc[r][2 * i], acc[r][2 * i + 1], a.bias, a.actq, a.acts, g, e, it, (prow0 >> 5) + rgl, lane);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
      const int m0 = 4 * (lane >> 5);
#pragma unroll
      for (int r = 0; r < RW; r++) {
        const int rgl = wr * RW + r;
        if (rgl * 32 >= nrows) continue;
        // rows 8*jj + m0 + i of the row group: four runs of four consecutive rows
        int32_t pr[16];
        float wt[16];
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
          const int row = rgl * 32 + 8 * jj + m0;
          const int4 p4 = *reinterpret_cast<const int4*>(a.prow_pair + prow0 + row);
          const f32x4_t w4 = *reinterpret_cast<const f32x4_t*>(a.prow_w + prow0 + row);
          pr[4 * jj] = row < nrows ? p4.x : -1;
          pr[4 * jj + 1] = row + 1 < nrows ? p4.y : -1;
          pr[4 * jj + 2] = row + 2 < nrows ? p4.z : -1;
          pr[4 * jj + 3] = row + 3 < nrows ? p4.w : -1;
#pragma unroll
          for (int i = 0; i < 4; i++) wt[4 * jj + i] = w4[i];
        }
#pragma unroll
        for (int j = 0; j < CW; j++) {
          const int64_t nt = (int64_t)x * NT + wc * CW + j;
          if (nt < g.nht) {
            const int64_t col = nt * 32 + (lane & 31);
            const float bb = a.bias ? bf16_bits_to_f32(a.bias[(int64_t)e * g.H + col]) : 0.f;
#pragma unroll
            for (int q = 0; q < 16; q++)
              if (pr[q] >= 0) a.obuf[(int64_t)pr[q] * g.H + col] = wt[q] * (acc[r][j][q] + bb);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }
}

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ obuf, uint16_t* __restrict__ y,
                                                      int64_t H8, int k, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / H8, c = i - t * H8;
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    const f32x4_t* src = reinterpret_cast<const f32x4_t*>(obuf) + ((t * k) * H8 + c) * 2;
    for (int j = 0; j < k; j++) {
      s0 += __builtin_nontemporal_load(src + j * H8 * 2);
      s1 += __builtin_nontemporal_load(src + j * H8 * 2 + 1);
    }
    u32x4_t o;
    o[0] = f32_to_bf16_bits(s0[0]) | (f32_to_bf16_bits(s0[1]) << 16);
    o[1] = f32_to_bf16_bits(s0[2]) | (f32_to_bf16_bits(s0[3]) << 16);
    o[2] = f32_to_bf16_bits(s1[0]) | (f32_to_bf16_bits(s1[1]) << 16);
    o[3] = f32_to_bf16_bits(s1[2]) | (f32_to_bf16_bits(s1[3]) << 16);
    reinterpret_cast<u32x4_t*>(y)[i] = o;
  }
}

template <bool G1, int WR, int WC, int RW, int CW, int D>
int launch_cfg(const GemmArgs& a, int64_t max_tiles, int wg_per_cu, hipStream_t stream) {
  using C = Cfg<WR, WC, RW, CW, D>;
  const int64_t nx = (G1 ? a.g.ncb1 : a.g.ncb2) * kCB / C::NT;
  int64_t items = max_tiles * nx;
  int64_t grid = 256 * wg_per_cu;
  if (items < grid) grid = items;
  grid = kXcds * cdiv(grid, kXcds);
  if (grid < kXcds) grid = kXcds;
  hipLaunchKernelGGL((grouped_gemm_kernel<G1, WR, WC, RW, CW, D>), dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError() == hipSuccess ? MXFP4_OK : MXFP4_ERR_DEVICE;
}

}  // namespace

// Tile configurations by rows per M tile (32 * NRG): 1 row group for decode-like loads, 2 or 4 for
// larger ones.  The first GEMM covers a whole column block per workgroup; the 128-row second GEMM
// covers half of one so that two workgroups share a CU and one's output stores overlap the other's
// MFMAs.
int launch_gemm1(int NRG, const GemmArgs& a, int64_t max_tiles, hipStream_t stream) {
  switch (NRG) {
    case 1: return launch_cfg<true, 1, 4, 1, 4, 3>(a, max_tiles, 2, stream);
    case 2: return launch_cfg<true, 1, 4, 2, 4, 3>(a, max_tiles, 2, stream);
    case 4: return launch_cfg<true, 2, 2, 2, 8, 5>(a, max_tiles, 1, stream);
    default: return MXFP4_ERR_SHAPE;
  }
}

int launch_gemm2(int NRG, const GemmArgs& a, int64_t max_tiles, hipStream_t stream) {
  switch (NRG) {
    case 1: return launch_cfg<false, 1, 4, 1, 4, 3>(a, max_tiles, 2, stream);
    case 2: return launch_cfg<false, 1, 4, 2, 4, 3>(a, max_tiles, 2, stream);
    case 4: return launch_cfg<false, 2, 2, 2, 4, 3>(a, max_tiles, 2, stream);
    default: return MXFP4_ERR_SHAPE;
  }
}

int launch_combine(const float* obuf, void* y, int64_t T, int64_t H, int k, hipStream_t stream) {
  const int64_t n = T * (H / 8);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (n > 0)
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, obuf, (uint16_t*)y, H / 8, k, n);
  return hipGetLastError() == hipSuccess ? MXFP4_OK : MXFP4_ERR_DEVICE;
}
