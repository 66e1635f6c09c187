// Grouped expert GEMMs of the MoE layer on gfx950 block-scaled MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4), with the SwiGLU and the weighted scatter-combine fused into
// their epilogues.
//
// [NS: grouped w13 GEMM, SwiGLU = silu(w1 half) * (w3 half), grouped w2 GEMM, weighted top-k combine;
//  MXFP4 weights with E8M0 scales per 32 elements; P1 Implementation breakdown: the mixed-input fused
//  MoE multiplies packed 4-bit weights with per-32 group scales by 16-bit activations]
//
// The MFMA has no bf16 operand, so a bf16 activation enters as three E2M3 (FP6) terms x = t0 + t1 + t2,
// each with its own E8M0 scale per 32 elements, and every product is issued once per term against the
// same FP4 weight registers.  FP6 x FP4 runs at the FP4 rate on gfx950.  Two terms keep only about
// eight bits relative to the block maximum, which is not enough for the elementwise tolerance on
// millions of outputs; three terms leave the bf16 rounding of the activation as the largest error.
//
// First GEMM, transposed: D[n][m] = sum_k W13[n][k] x[m][k], weights as the A operand (rows n = 32
// gate or up rows of one 32-column tile), tokens as the B operand (columns m = 32 tokens gathered from
// the sorted pair list).  Lane l of the 32x32 result holds token l%32 and rows 8*jj + 4*(l/32) + i, so
// gate and up of one column sit in the same lane (SwiGLU in registers) and a 32-element block of the
// activation is split over the two lane halves (one exchange for the block maximum).
//
// Second GEMM, not transposed: D[m][n] = sum_k act[m][k] W2[n][k]; lane l holds output column l%32 and
// rows 8*jj + 4*(l/32) + i, so each fp32 atomic instruction adds 2 x 32 consecutive floats.
#include <type_traits>

#include "common.h"

namespace {

typedef decltype(__builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(bf16x32_t{}, 1.0f)) fp6x32_t;

MX_DEV u32x4_t ld16(const uint8_t* p) { return *reinterpret_cast<const u32x4_t*>(p); }

MX_DEV i32x8_t fp4_operand(u32x4_t v) {
  return i32x8_t{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
}
// One operand slot (kSlot bytes): the three E2M3 terms, 6 dwords each, back to back.
MX_DEV void fp6_term_operands(const uint8_t* p, i32x8_t* o) {
  const u32x4_t a = ld16(p), b = ld16(p + 16), c = ld16(p + 32), d = ld16(p + 48), f = ld16(p + 64);
  o[0] = i32x8_t{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], 0, 0};
  o[1] = i32x8_t{(int)b[2], (int)b[3], (int)c[0], (int)c[1], (int)c[2], (int)c[3], 0, 0};
  o[2] = i32x8_t{(int)d[0], (int)d[1], (int)d[2], (int)d[3], (int)f[0], (int)f[1], 0, 0};
}

constexpr int kFp4 = 4, kFp6 = 2;  // MFMA operand format codes (E2M1, E2M3)

template <int MT>
struct G1Acc {
  f32x16_t g[MT], u[MT];
};

MX_DEV float silu(float g) { return g / (1.0f + __expf(-g)); }

// First GEMM epilogue for one (32-column activation tile `it`, row group `rg`) result held by one
// wave: bias, SwiGLU in fp32, then the three-term E2M3 split of each 32-element block (one block = the
// two lane halves of a token column; each block maximum needs one exchange across the halves), written
// in the second GEMM's operand layout.  The last K tile of the second GEMM is completed with a zero
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
  uint8_t* chunk = actq + ((rg * g.nkt2 + kt2) * 64 + kb * 32 + m) * kSlot;
  uint8_t* sc = acts + ((rg * g.ngrp2 + (kt2 >> 2)) * 64 + kb * 32 + m) * (kTerms * 4) + (kt2 & 3);
  // Each term quantizes the bf16 rounding of the fp32 remainder; the remainder itself stays fp32
  // (subtracting a term, a multiple of the remainder's ulp within one grid step, is exact in fp32).
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
    if (h == 0) sc[term * 4] = (uint8_t)ex;
    if (term + 1 < kTerms) {
      const auto deq = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(codes, sv);
#pragma unroll
      for (int q = 0; q < 16; q++) cur[q] = cur[q] - deq[q];
    }
  }
  if ((it == g.nit - 1) && (g.nit & 1)) {
    uint32_t* zp = reinterpret_cast<uint32_t*>(actq + ((rg * g.nkt2 + kt2) * 64 + 32 + m) * kSlot + h * (kSlot / 2));
#pragma unroll
    for (int q = 0; q < kSlot / 8; q++) zp[q] = 0;
    if (h == 0) {
      uint8_t* zs = acts + ((rg * g.ngrp2 + (kt2 >> 2)) * 64 + 32 + m) * (kTerms * 4) + (kt2 & 3);
#pragma unroll
      for (int term = 0; term < kTerms; term++) zs[term * 4] = 0;
    }
  }
}

template <int MT>
MX_DEV void g1_epilogue(const G1Acc<MT>& acc, const uint16_t* __restrict__ b13, uint8_t* __restrict__ actq,
                        uint8_t* __restrict__ acts, const MoeGeom& g, int e, int64_t it, int prow0, int nvg, int lane) {
#pragma unroll
  for (int mt = 0; mt < MT; mt++)
    if (mt < nvg) g1_epilogue_tile(acc.g[mt], acc.u[mt], b13, actq, acts, g, e, it, (prow0 >> 5) + mt, lane);
}

// ------------------------------------------------------------------------------------------------
// First GEMM + SwiGLU + three-term split of the activation.
//
// Workgroup: NW waves; wave w owns the 32 activation columns of tile it = blockIdx.x*NW + w (its gate
// and up weight rows, 2 x 32) against the MT*32 tokens of one M tile.  The token operand of each 64-K
// step is shared by all waves, so the workgroup stages it in LDS (double-buffered): thread t copies
// 16-byte pieces of the gathered three-term rows, and each wave then reads its MFMA operands (one slot per lane)
// from LDS.  The weight operand is private to the wave and is loaded straight from global memory one
// K step ahead.  One barrier per K step.  grid: x = column tiles / NW, y = M tiles (strided loop).
template <int MT, int NW>
struct G1Smem {
  uint8_t b[2][MT * 64 * kSlot];
  int32_t tok[MT * 32];
};

// DEEP (used for single-row-group tiles, i.e. decode shapes): the weight operand of the next group of
// four K steps is requested while the current group computes, so each wave keeps 8 KB of weights in
// flight -- the weight stream is the bound there.  Otherwise one K step ahead (fewer registers).
template <int MT, int NW, bool DEEP>
__global__ __launch_bounds__(NW * 64) void gemm1_kernel(const uint8_t* __restrict__ w13q, const uint32_t* __restrict__ w13s,
                                                         const uint16_t* __restrict__ b13, const uint8_t* __restrict__ xq,
                                                         const uint8_t* __restrict__ xs,
                                                         const int32_t* __restrict__ prow_pair,
                                                         const int4* __restrict__ tiles, const int32_t* __restrict__ ntiles,
                                                         uint8_t* __restrict__ actq, uint8_t* __restrict__ acts, MoeGeom g,
                                                         int k) {
  __shared__ G1Smem<MT, NW> sm;
  constexpr int kThreads = NW * 64;
  constexpr int kChunks = MT * 64 * (kSlot / 16);  // 16-byte pieces of one staged token tile
  constexpr int kPer = (kChunks + kThreads - 1) / kThreads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t it_raw = (int64_t)blockIdx.x * NW + wave;
  const bool active = it_raw < g.nit;  // wave-uniform; inactive waves only help with loads and barriers
  const int64_t it = active ? it_raw : 0;
  const int64_t nblk1 = 2 * g.nkt1;
  const int nt_all = *ntiles;

  for (int tile = blockIdx.y; tile < nt_all; tile += gridDim.y) {
    const int4 td = tiles[tile];
    const int e = td.x, prow0 = td.y, nrows = td.z;
    const int nvg = (nrows + 31) >> 5;
    __syncthreads();  // the previous tile's readers are done with sm
    for (int r = tid; r < MT * 32; r += kThreads) {
      int tok = 0;
      if (r < nrows) {
        const int pair = prow_pair[prow0 + r];
        if (pair >= 0) tok = pair / k;
      }
      sm.tok[r] = tok;
    }
    __syncthreads();

    const uint8_t* src[kPer];
    int dst[kPer];
    bool live[kPer];
#pragma unroll
    for (int i = 0; i < kPer; i++) {
      const int c = tid + i * kThreads;
      const int slot = c / (kSlot / 16), part = c - (kSlot / 16) * slot;
      const int mt = slot >> 6, ln = slot & 63;
      live[i] = c < kChunks && mt < nvg;
      const int tok = live[i] ? sm.tok[mt * 32 + (ln & 31)] : 0;
      src[i] = xq + ((int64_t)tok * nblk1 + (ln >> 5)) * kSlot + part * 16;
      dst[i] = slot * kSlot + part * 16;
    }
    const uint8_t* xsrow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
      xsrow[mt] = xs + (int64_t)sm.tok[mt * 32 + (lane & 31)] * g.ngrp1 * (kTerms * 8) + (lane >> 5) * 4;
    const uint8_t* wa = w13q + ((int64_t)e * g.nit + it) * g.nkt1 * 2048 + lane * 16;
    const uint32_t* wsa = w13s + ((int64_t)e * g.nit + it) * g.ngrp1 * 128 + lane;

    G1Acc<MT> acc;
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
      for (int i = 0; i < 16; i++) { acc.g[mt][i] = 0.f; acc.u[mt][i] = 0.f; }

    // prologue: K step 0
    {
      u32x4_t stage[kPer];
#pragma unroll
      for (int i = 0; i < kPer; i++)
        if (live[i]) stage[i] = ld16(src[i]);
#pragma unroll
      for (int i = 0; i < kPer; i++)
        if (live[i]) *reinterpret_cast<u32x4_t*>(&sm.b[0][dst[i]]) = stage[i];
    }
    u32x4_t ag = {0u, 0u, 0u, 0u}, au = {0u, 0u, 0u, 0u};
    u32x4_t cg[4], cu[4];  // DEEP: weights of the current group of K steps
    if (active) {
      if constexpr (DEEP) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
          if (j < g.nkt1) {
            cg[j] = ld16(wa + j * 2048);
            cu[j] = ld16(wa + j * 2048 + 1024);
          }
        }
      } else {
        ag = ld16(wa);
        au = ld16(wa + 1024);
      }
    }
    __syncthreads();

    for (int64_t grp = 0; grp < g.ngrp1; grp++) {
      u32x4_t ng[4], nu[4];
      if constexpr (DEEP) {
        if (active && grp + 1 < g.ngrp1) {
#pragma unroll
          for (int j = 0; j < 4; j++) {
            const int64_t kn = (grp + 1) * 4 + j;
            if (kn < g.nkt1) {
              ng[j] = ld16(wa + kn * 2048);
              nu[j] = ld16(wa + kn * 2048 + 1024);
            }
          }
        }
      }
      uint32_t sg = 0, su = 0;
      uint32_t sx[MT][kTerms];
      if (active) {
        sg = wsa[grp * 128];
        su = wsa[grp * 128 + 64];
#pragma unroll
        for (int mt = 0; mt < MT; mt++)
#pragma unroll
          for (int term = 0; term < kTerms; term++)
            sx[mt][term] = *reinterpret_cast<const uint32_t*>(xsrow[mt] + grp * (kTerms * 8) + term * 8);
      }
      auto step = [&](auto jc) {
        constexpr int J = decltype(jc)::value;
        const int64_t kt = grp * 4 + J;
        const bool more = kt + 1 < g.nkt1;
        u32x4_t stage[kPer];
        u32x4_t ag_n = ag, au_n = au;
        if (more) {
#pragma unroll
          for (int i = 0; i < kPer; i++)
            if (live[i]) stage[i] = ld16(src[i] + (kt + 1) * (2 * kSlot));
          if constexpr (!DEEP) {
            if (active) {
              ag_n = ld16(wa + (kt + 1) * 2048);
              au_n = ld16(wa + (kt + 1) * 2048 + 1024);
            }
          }
        }
        if (active) {
          const i32x8_t a_g = fp4_operand(DEEP ? cg[J] : ag), a_u = fp4_operand(DEEP ? cu[J] : au);
          const uint8_t* bb = sm.b[kt & 1];
#pragma unroll
          for (int mt = 0; mt < MT; mt++) {
            if (mt < nvg) {
              i32x8_t bt[kTerms];
              fp6_term_operands(bb + (mt * 64 + lane) * kSlot, bt);
#pragma unroll
              for (int term = 0; term < kTerms; term++) {
                acc.g[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a_g, bt[term], acc.g[mt], kFp4, kFp6, J, sg, J,
                                                                            sx[mt][term]);
                acc.u[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a_u, bt[term], acc.u[mt], kFp4, kFp6, J, su, J,
                                                                            sx[mt][term]);
              }
            }
          }
        }
        if (more) {
#pragma unroll
          for (int i = 0; i < kPer; i++)
            if (live[i]) *reinterpret_cast<u32x4_t*>(&sm.b[(kt + 1) & 1][dst[i]]) = stage[i];
        }
        __syncthreads();
        ag = ag_n;
        au = au_n;
      };
      step(std::integral_constant<int, 0>{});
      if (grp * 4 + 1 < g.nkt1) step(std::integral_constant<int, 1>{});
      if (grp * 4 + 2 < g.nkt1) step(std::integral_constant<int, 2>{});
      if (grp * 4 + 3 < g.nkt1) step(std::integral_constant<int, 3>{});
      if constexpr (DEEP) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
          cg[j] = ng[j];
          cu[j] = nu[j];
        }
      }
    }
    if (active) g1_epilogue<MT>(acc, b13, actq, acts, g, e, it, prow0, nvg, lane);
  }
}

// ------------------------------------------------------------------------------------------------
// Second GEMM + bias + routing weight.  Workgroup: NW waves over NW column tiles of 32 (of H) and one
// M tile; the activation tile (MT row groups, contiguous 3 KB per row group and K step) is staged in
// LDS, double-buffered; the weight operand is private per wave and prefetched one K step ahead.  The
// epilogue writes w * (o + b2) as bf16 to o_buf[pair][H] (token-major), and combine_kernel sums the k
// rows of each token: no atomics, a fixed summation order.
template <int MT, int NW, bool DEEP>
__global__ __launch_bounds__(NW * 64) void gemm2_kernel(const uint8_t* __restrict__ w2q, const uint32_t* __restrict__ w2s,
                                                         const uint16_t* __restrict__ b2, const uint8_t* __restrict__ actq,
                                                         const uint8_t* __restrict__ acts,
                                                         const int32_t* __restrict__ prow_pair,
                                                         const float* __restrict__ topw, const int4* __restrict__ tiles,
                                                         const int32_t* __restrict__ ntiles, float* __restrict__ obuf,
                                                         MoeGeom g, int k) {
  constexpr int kTileBytes = 64 * kSlot;  // one row group's operand for one K step
  __shared__ uint8_t sa[2][MT * kTileBytes];
  __shared__ int32_t s_pair[MT * 32];
  __shared__ float s_w[MT * 32];
  constexpr int kThreads = NW * 64;
  constexpr int kChunks = MT * (kTileBytes / 16);
  constexpr int kPer = (kChunks + kThreads - 1) / kThreads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nt_raw = (int64_t)blockIdx.x * NW + wave;
  const bool active = nt_raw < g.nht;
  const int64_t nt = active ? nt_raw : 0;
  const int nt_all = *ntiles;

  for (int tile = blockIdx.y; tile < nt_all; tile += gridDim.y) {
    const int4 td = tiles[tile];
    const int e = td.x, prow0 = td.y, nrows = td.z;
    const int nvg = (nrows + 31) >> 5;
    const int64_t rg0 = prow0 >> 5;
    __syncthreads();  // the previous tile's readers are done with sa, s_pair, s_w
    for (int r = tid; r < MT * 32; r += kThreads) {
      int pair = -1;
      float wt = 0.f;
      if (r < nrows) {
        pair = prow_pair[prow0 + r];
        if (pair >= 0) wt = topw[pair];
      }
      s_pair[r] = pair;
      s_w[r] = wt;
    }

    const uint8_t* src[kPer];
    int dst[kPer];
    bool live[kPer];
#pragma unroll
    for (int i = 0; i < kPer; i++) {
      const int c = tid + i * kThreads;
      const int mt = c / (kTileBytes / 16), off = (c - (kTileBytes / 16) * mt) * 16;
      live[i] = c < kChunks && mt < nvg;
      src[i] = actq + (rg0 + (live[i] ? mt : 0)) * g.nkt2 * kTileBytes + off;
      dst[i] = mt * kTileBytes + off;
    }
    const uint8_t* sarow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++) sarow[mt] = acts + ((rg0 + mt) * g.ngrp2 * 64 + lane) * (kTerms * 4);
    const uint8_t* wb = w2q + ((int64_t)e * g.nht + nt) * g.nkt2 * 1024 + lane * 16;
    const uint32_t* wsb = w2s + ((int64_t)e * g.nht + nt) * g.ngrp2 * 64 + lane;

    f32x16_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
      for (int i = 0; i < 16; i++) acc[mt][i] = 0.f;

    {
      u32x4_t stage[kPer];
#pragma unroll
      for (int i = 0; i < kPer; i++)
        if (live[i]) stage[i] = ld16(src[i]);
#pragma unroll
      for (int i = 0; i < kPer; i++)
        if (live[i]) *reinterpret_cast<u32x4_t*>(&sa[0][dst[i]]) = stage[i];
    }
    u32x4_t wv = {0u, 0u, 0u, 0u};
    u32x4_t cw[4];  // DEEP: weights of the current group of K steps
    if (active) {
      if constexpr (DEEP) {
#pragma unroll
        for (int j = 0; j < 4; j++)
          if (j < g.nkt2) cw[j] = ld16(wb + j * 1024);
      } else {
        wv = ld16(wb);
      }
    }
    __syncthreads();

    for (int64_t grp = 0; grp < g.ngrp2; grp++) {
      u32x4_t nw[4];
      if constexpr (DEEP) {
        if (active && grp + 1 < g.ngrp2) {
#pragma unroll
          for (int j = 0; j < 4; j++) {
            const int64_t kn = (grp + 1) * 4 + j;
            if (kn < g.nkt2) nw[j] = ld16(wb + kn * 1024);
          }
        }
      }
      uint32_t sb = 0;
      uint32_t sa_t[MT][kTerms];
      if (active) {
        sb = wsb[grp * 64];
#pragma unroll
        for (int mt = 0; mt < MT; mt++)
#pragma unroll
          for (int term = 0; term < kTerms; term++)
            sa_t[mt][term] = mt < nvg ? *reinterpret_cast<const uint32_t*>(sarow[mt] + grp * (64 * kTerms * 4) + term * 4) : 0u;
      }
      auto step = [&](auto jc) {
        constexpr int J = decltype(jc)::value;
        const int64_t kt = grp * 4 + J;
        const bool more = kt + 1 < g.nkt2;
        u32x4_t stage[kPer];
        u32x4_t wv_n = wv;
        if (more) {
#pragma unroll
          for (int i = 0; i < kPer; i++)
            if (live[i]) stage[i] = ld16(src[i] + (kt + 1) * kTileBytes);
          if constexpr (!DEEP) {
            if (active) wv_n = ld16(wb + (kt + 1) * 1024);
          }
        }
        if (active) {
          const i32x8_t bw = fp4_operand(DEEP ? cw[J] : wv);
          const uint8_t* ab = sa[kt & 1];
#pragma unroll
          for (int mt = 0; mt < MT; mt++) {
            if (mt < nvg) {
              i32x8_t at[kTerms];
              fp6_term_operands(ab + mt * kTileBytes + lane * kSlot, at);
#pragma unroll
              for (int term = 0; term < kTerms; term++)
                acc[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(at[term], bw, acc[mt], kFp6, kFp4, J, sa_t[mt][term],
                                                                          J, sb);
            }
          }
        }
        if (more) {
#pragma unroll
          for (int i = 0; i < kPer; i++)
            if (live[i]) *reinterpret_cast<u32x4_t*>(&sa[(kt + 1) & 1][dst[i]]) = stage[i];
        }
        __syncthreads();
        wv = wv_n;
      };
      step(std::integral_constant<int, 0>{});
      if (grp * 4 + 1 < g.nkt2) step(std::integral_constant<int, 1>{});
      if (grp * 4 + 2 < g.nkt2) step(std::integral_constant<int, 2>{});
      if (grp * 4 + 3 < g.nkt2) step(std::integral_constant<int, 3>{});
      if constexpr (DEEP) {
#pragma unroll
        for (int j = 0; j < 4; j++) cw[j] = nw[j];
      }
    }

    if (active) {
      const int64_t col = nt * 32 + (lane & 31);
      const float bias = b2 ? bf16_bits_to_f32(b2[(int64_t)e * g.H + col]) : 0.f;
      const int h = lane >> 5;
#pragma unroll
      for (int mt = 0; mt < MT; mt++) {
        if (mt >= nvg) continue;
#pragma unroll
        for (int q = 0; q < 16; q++) {
          const int r = mt * 32 + 8 * (q >> 2) + 4 * h + (q & 3);
          const int pair = s_pair[r];
          if (pair >= 0) obuf[(int64_t)pair * g.H + col] = s_w[r] * (acc[mt][q] + bias);
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------------------
// Row-split kernels for M tiles of WM row groups (prefill shapes).  Wave w owns row group w of the
// tile; the workgroup shares the weight tiles of each 64-K step.  Every operand of a K step -- the
// weight tiles and their scale registers, each wave's activation slots and their scale registers --
// is copied global -> LDS by the gfx950 direct loads (global_load_lds_dwordx4 / _dword: lane i of a
// wave writes base + i*size), into a ring of D stages, so D-1 steps of loads are in flight while a
// step computes and no registers are spent on staging.  Each wave waits for its own copies with an
// exact vmcnt (the same number of copies per wave and step, dummy-but-valid addresses included), then
// one workgroup barrier makes every wave's copies of that step visible and frees the stage read in
// the previous step, which is refilled right after the barrier.  Every weight fragment read from LDS
// feeds three MFMAs (one per activation term), every activation fragment feeds all weight tiles.

typedef __attribute__((address_space(3))) void* lds_vptr_t;

MX_DEV void dma16(const void* g, uint8_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_vptr_t)lds_wave_base, 16, 0, 0);
}
MX_DEV void dma4(const void* g, uint8_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_vptr_t)lds_wave_base, 4, 0, 0);
}
// s_waitcnt with vmcnt <= N and no wait on the other counters (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt 6:4 = 7, lgkmcnt 11:8 = 15).
template <int N>
MX_DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x70 | 0xF00);
}
MX_DEV void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// Workgroup barrier without the release/acquire fence of __syncthreads (which would wait for every
// outstanding copy); the asm statements keep the compiler from moving LDS accesses across it.
MX_DEV void block_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// Wait until at most c (0..D-2) later stages of kOps copies each are still in flight.
template <int kOps, int D>
MX_DEV void wait_stage(int c) {
  static_assert(D >= 2 && D <= 5, "ring depth");
  if (c >= 3) wait_vmcnt<kOps * (D - 2 >= 3 ? 3 : 0)>();
  else if (c == 2) wait_vmcnt<kOps * (D - 2 >= 2 ? 2 : 0)>();
  else if (c == 1) wait_vmcnt<kOps>();
  else wait_vmcnt<0>();
}

// XCD-aware work split for the row-split kernels.  Workgroups are dispatched round-robin over the
// MI355X's 8 XCDs (workgroup b runs on XCD b % 8) and each XCD has its own L2.  The (M tile, column
// block) items are given to XCDs in contiguous ranges, column block fastest, so the column blocks of
// one M tile (which read the same gathered activations) and the M tiles of one expert (which read the
// same weights) run on the same XCD at about the same time.  Returns false when this workgroup has no
// item.  The grid must hold at least 8 * ceil(max_tiles * nx / 8) workgroups.
constexpr int kXcds = 8;
MX_DEV bool xcd_item(int nt_all, int nx, int& tile, int& x) {
  const int64_t total = (int64_t)nt_all * nx;
  const int64_t chunk = (total + kXcds - 1) / kXcds;
  const int64_t b = blockIdx.x;
  const int64_t local = b / kXcds;
  const int64_t p = (b % kXcds) * chunk + local;
  if (local >= chunk || p >= total) return false;
  tile = (int)(p / nx);
  x = (int)(p % nx);
  return true;
}

// First GEMM: the workgroup covers NACT activation tiles (2*NACT gate/up weight tiles of 32 rows).
template <int WM, int NACT, int D>
__global__ __launch_bounds__(WM * 64) void gemm1_rows_kernel(
    const uint8_t* __restrict__ w13q, const uint32_t* __restrict__ w13s, const uint16_t* __restrict__ b13,
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, const int32_t* __restrict__ prow_pair,
    const int4* __restrict__ tiles, const int32_t* __restrict__ ntiles, uint8_t* __restrict__ actq,
    uint8_t* __restrict__ acts, MoeGeom g, int k) {
  constexpr int NWT = 2 * NACT;  // weight tiles: 2i = gate of activation tile i, 2i+1 = its up
  static_assert(NWT % WM == 0, "weight tiles split evenly over waves");
  constexpr int WPW = NWT / WM;
  constexpr int kParts = kSlot / 16;
  constexpr int oW = 0, oWS = NWT * 1024, oX = oWS + NWT * 256, oXS = oX + WM * kParts * 1024;
  constexpr int kStage = oXS + WM * kTerms * 256;
  constexpr int kOps = 2 * WPW + kParts + kTerms;  // copies per wave per K step
  __shared__ __attribute__((aligned(16))) uint8_t smem[D * kStage];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nblk1 = 2 * g.nkt1;
  const int64_t nkt = g.nkt1;
  int tile, xb;
  if (!xcd_item(*ntiles, (int)((g.nit + NACT - 1) / NACT), tile, xb)) return;
  const int64_t it0 = (int64_t)xb * NACT;
  {
    const int4 td = tiles[tile];
    const int e = td.x, prow0 = td.y, nrows = td.z;
    const bool valid = wave * 32 < nrows;  // wave-uniform
    // Copies of the wave's 32 gathered rows go by contiguous runs: per K step a row holds two slots
    // (160 B, kParts*2 chunks of 16 B) and 6 scale words (24 B), so chunk c of the wave's step data is
    // row c / (2*kParts), part c % (2*kParts), and lane l of copy i takes chunk i*64 + l.  The LDS
    // image is row-major: slot of (row m, block parity kb) at (m*2*kParts + kb*kParts)*16.
    const uint8_t* xsrc[kParts];
    const uint8_t* xssrc[kTerms];
#pragma unroll
    for (int i = 0; i < kParts; i++) {
      const int c = i * 64 + lane;
      const int rr = wave * 32 + c / (2 * kParts);
      int tk = 0;
      if (rr < nrows) {
        const int pair = prow_pair[prow0 + rr];
        if (pair >= 0) tk = pair / k;
      }
      xsrc[i] = xq + (int64_t)tk * nblk1 * kSlot + (c % (2 * kParts)) * 16;
    }
#pragma unroll
    for (int i = 0; i < kTerms; i++) {
      const int c = i * 64 + lane;
      const int rr = wave * 32 + c / (2 * kTerms);
      int tk = 0;
      if (rr < nrows) {
        const int pair = prow_pair[prow0 + rr];
        if (pair >= 0) tk = pair / k;
      }
      xssrc[i] = xs + (int64_t)tk * g.ngrp1 * (kTerms * 8) + (c % (2 * kTerms)) * 4;
    }
    const uint8_t* wsrc[WPW];
    const uint32_t* wssrc[WPW];
#pragma unroll
    for (int i = 0; i < WPW; i++) {
      const int j = wave * WPW + i;
      const int64_t itj = it0 + (j >> 1);
      const int64_t itc = itj < g.nit ? itj : it0;  // valid address; the tile's MFMAs are skipped
      wsrc[i] = w13q + (((int64_t)e * g.nit + itc) * g.nkt1 * 2 + (j & 1)) * 1024 + lane * 16;
      wssrc[i] = w13s + ((int64_t)e * g.nit + itc) * g.ngrp1 * 128 + (j & 1) * 64 + lane;
    }
    auto issue = [&](int64_t kt, int stage) {
      uint8_t* base = smem + stage * kStage;
#pragma unroll
      for (int i = 0; i < WPW; i++) dma16(wsrc[i] + kt * 2048, base + oW + (wave * WPW + i) * 1024);
#pragma unroll
      for (int i = 0; i < WPW; i++) dma4(wssrc[i] + (kt >> 2) * 128, base + oWS + (wave * WPW + i) * 256);
#pragma unroll
      for (int i = 0; i < kParts; i++) dma16(xsrc[i] + kt * (2 * kSlot), base + oX + (wave * kParts + i) * 1024);
#pragma unroll
      for (int i = 0; i < kTerms; i++) dma4(xssrc[i] + (kt >> 2) * (kTerms * 8), base + oXS + (wave * kTerms + i) * 256);
    };

    f32x16_t acc[NWT];
#pragma unroll
    for (int j = 0; j < NWT; j++)
#pragma unroll
      for (int i = 0; i < 16; i++) acc[j][i] = 0.f;

    wait_vmcnt<0>();  // nothing of the previous tile still in flight
    block_sync();     // every wave is done reading the ring
#pragma unroll
    for (int s = 0; s < D - 1; s++)
      if (s < nkt) issue(s, s);

    // Operand fragments of one K step, read from LDS one step ahead of the MFMAs that use them.
    struct Frag {
      u32x4_t a[NWT];
      uint32_t sa[NWT];
      u32x4_t x[kParts];
      uint32_t sx[kTerms];
    };
    auto load_frag = [&](int64_t kt, Frag& f) {
      const uint8_t* base = smem + (kt % D) * kStage;
      const uint8_t* xb = base + oX + wave * kParts * 1024 + ((lane & 31) * 2 * kParts + (lane >> 5) * kParts) * 16;
#pragma unroll
      for (int q = 0; q < kParts; q++) f.x[q] = ld16(xb + q * 16);
#pragma unroll
      for (int t = 0; t < kTerms; t++)
        f.sx[t] = *reinterpret_cast<const uint32_t*>(base + oXS + (wave * kTerms) * 256 +
                                                     ((lane & 31) * 2 * kTerms + t * 2 + (lane >> 5)) * 4);
#pragma unroll
      for (int j = 0; j < NWT; j++) {
        f.a[j] = ld16(base + oW + j * 1024 + lane * 16);
        f.sa[j] = *reinterpret_cast<const uint32_t*>(base + oWS + j * 256 + lane * 4);
      }
    };
    // Make stage kt visible to every wave (own copies counted by vmcnt, then the barrier), after which
    // the ring slot of stage kt - 1 is free: refill it with stage kt + D - 1.
    auto arrive = [&](int64_t kt) {
      const int64_t ahead = nkt - 1 - kt;
      wait_stage<kOps, D>((int)(ahead < D - 2 ? ahead : D - 2));
      wait_lgkmcnt0();
      block_sync();
      if (kt + D - 1 < nkt) issue(kt + D - 1, (int)((kt + D - 1) % D));
    };

    auto kloop = [&](auto fullc) {
      constexpr bool FULL = decltype(fullc)::value;
      // Waves without rows (a short last M tile) run the same instruction stream on harmless data and
      // skip the epilogue: keeping the loop free of divergent branches lets the compiler wait for exactly
      // the LDS reads each MFMA needs instead of draining all of them.
      Frag cur, nxt;
      arrive(0);
      load_frag(0, cur);
      for (int64_t grp = 0; grp < g.ngrp1; grp++) {
        auto step = [&](auto jc) {
          constexpr int J = decltype(jc)::value;
          const int64_t kt = grp * 4 + J;
          const bool more = kt + 1 < nkt;
          // The MFMAs of step kt follow the reads of step kt + 1 in the same basic block, so they do not
          // wait for those reads.
          auto mfmas = [&]() {
          {
            i32x8_t bt[kTerms];
            bt[0] = i32x8_t{(int)cur.x[0][0], (int)cur.x[0][1], (int)cur.x[0][2], (int)cur.x[0][3], (int)cur.x[1][0],
                            (int)cur.x[1][1], 0, 0};
            bt[1] = i32x8_t{(int)cur.x[1][2], (int)cur.x[1][3], (int)cur.x[2][0], (int)cur.x[2][1], (int)cur.x[2][2],
                            (int)cur.x[2][3], 0, 0};
            bt[2] = i32x8_t{(int)cur.x[3][0], (int)cur.x[3][1], (int)cur.x[3][2], (int)cur.x[3][3], (int)cur.x[4][0],
                            (int)cur.x[4][1], 0, 0};
            // term-major: consecutive MFMAs use different accumulators
#pragma unroll
            for (int t = 0; t < kTerms; t++)
#pragma unroll
              for (int j = 0; j < NWT; j++)
                if (FULL || it0 + (j >> 1) < g.nit)
                  acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp4_operand(cur.a[j]), bt[t], acc[j], kFp4, kFp6,
                                                                           J, cur.sa[j], J, cur.sx[t]);
          }
          };
          if (more) {
            arrive(kt + 1);
            load_frag(kt + 1, nxt);
            mfmas();
            cur = nxt;
          } else {
            mfmas();
          }
        };
        step(std::integral_constant<int, 0>{});
        if (grp * 4 + 1 < nkt) step(std::integral_constant<int, 1>{});
        if (grp * 4 + 2 < nkt) step(std::integral_constant<int, 2>{});
        if (grp * 4 + 3 < nkt) step(std::integral_constant<int, 3>{});
      }
    };
    if (it0 + NACT <= g.nit) kloop(std::true_type{});
    else kloop(std::false_type{});
    if (valid) {
#pragma unroll
      for (int i = 0; i < NACT; i++)
        if (it0 + i < g.nit)
          g1_epilogue_tile(acc[2 * i], acc[2 * i + 1], b13, actq, acts, g, e, it0 + i, (prow0 >> 5) + wave, lane);
    }
  }
}

// Second GEMM: the workgroup covers NB column tiles of 32 (of H); w * (o + b2) goes to o_buf in fp32.
template <int WM, int NB, int D>
__global__ __launch_bounds__(WM * 64) void gemm2_rows_kernel(
    const uint8_t* __restrict__ w2q, const uint32_t* __restrict__ w2s, const uint16_t* __restrict__ b2,
    const uint8_t* __restrict__ actq, const uint8_t* __restrict__ acts, const int32_t* __restrict__ prow_pair,
    const float* __restrict__ topw, const int4* __restrict__ tiles, const int32_t* __restrict__ ntiles,
    float* __restrict__ obuf, MoeGeom g, int k) {
  static_assert(NB % WM == 0, "weight tiles split evenly over waves");
  constexpr int WPW = NB / WM;
  constexpr int kParts = kSlot / 16;
  constexpr int oW = 0, oWS = NB * 1024, oA = oWS + NB * 256, oAS = oA + WM * kParts * 1024;
  constexpr int kStage = oAS + WM * kTerms * 256;
  constexpr int kOps = 2 * WPW + kParts + kTerms;
  __shared__ __attribute__((aligned(16))) uint8_t smem[D * kStage];
  __shared__ int32_t s_pair[WM * 32];
  __shared__ float s_w[WM * 32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nkt = g.nkt2;
  int tile, xb;
  if (!xcd_item(*ntiles, (int)((g.nht + NB - 1) / NB), tile, xb)) return;
  const int64_t nt0 = (int64_t)xb * NB;
  {
    const int4 td = tiles[tile];
    const int e = td.x, prow0 = td.y, nrows = td.z;
    const bool valid = wave * 32 < nrows;
    const int64_t rg = (prow0 >> 5) + wave;  // inside the allocation even when not valid
    // The row group's operand chunk of a K step is contiguous (64 lane slots), so copy i takes bytes
    // [i*1024, (i+1)*1024) of it and the LDS image is the chunk itself; likewise the scale words.
    const uint8_t* achunk = actq + rg * g.nkt2 * 64 * kSlot + lane * 16;
    const uint8_t* schunk = acts + rg * g.ngrp2 * 64 * (kTerms * 4) + lane * 4;
    const uint8_t* wsrc[WPW];
    const uint32_t* wssrc[WPW];
#pragma unroll
    for (int i = 0; i < WPW; i++) {
      const int j = wave * WPW + i;
      const int64_t ntj = nt0 + j;
      const int64_t ntc = ntj < g.nht ? ntj : nt0;
      wsrc[i] = w2q + (((int64_t)e * g.nht + ntc) * g.nkt2) * 1024 + lane * 16;
      wssrc[i] = w2s + ((int64_t)e * g.nht + ntc) * g.ngrp2 * 64 + lane;
    }
    auto issue = [&](int64_t kt, int stage) {
      uint8_t* base = smem + stage * kStage;
#pragma unroll
      for (int i = 0; i < WPW; i++) dma16(wsrc[i] + kt * 1024, base + oW + (wave * WPW + i) * 1024);
#pragma unroll
      for (int i = 0; i < WPW; i++) dma4(wssrc[i] + (kt >> 2) * 64, base + oWS + (wave * WPW + i) * 256);
#pragma unroll
      for (int i = 0; i < kParts; i++) dma16(achunk + kt * (64 * kSlot) + i * 1024, base + oA + (wave * kParts + i) * 1024);
#pragma unroll
      for (int i = 0; i < kTerms; i++)
        dma4(schunk + (kt >> 2) * (64 * kTerms * 4) + i * 256, base + oAS + (wave * kTerms + i) * 256);
    };

    f32x16_t acc[NB];
#pragma unroll
    for (int j = 0; j < NB; j++)
#pragma unroll
      for (int i = 0; i < 16; i++) acc[j][i] = 0.f;

    wait_vmcnt<0>();
    block_sync();  // every wave is done with the ring, s_pair and s_w of the previous tile
    for (int rr = tid; rr < WM * 32; rr += WM * 64) {
      int pair = -1;
      float wt = 0.f;
      if (rr < nrows) {
        pair = prow_pair[prow0 + rr];
        if (pair >= 0) wt = topw[pair];
      }
      s_pair[rr] = pair;
      s_w[rr] = wt;
    }
#pragma unroll
    for (int s = 0; s < D - 1; s++)
      if (s < nkt) issue(s, s);

    struct Frag {
      u32x4_t b[NB];
      uint32_t sb[NB];
      u32x4_t x[kParts];
      uint32_t sa[kTerms];
    };
    auto load_frag = [&](int64_t kt, Frag& f) {
      const uint8_t* base = smem + (kt % D) * kStage;
      const uint8_t* ab = base + oA + wave * kParts * 1024 + lane * kSlot;
#pragma unroll
      for (int q = 0; q < kParts; q++) f.x[q] = ld16(ab + q * 16);
#pragma unroll
      for (int t = 0; t < kTerms; t++)
        f.sa[t] = *reinterpret_cast<const uint32_t*>(base + oAS + (wave * kTerms) * 256 + lane * (kTerms * 4) + t * 4);
#pragma unroll
      for (int j = 0; j < NB; j++) {
        f.b[j] = ld16(base + oW + j * 1024 + lane * 16);
        f.sb[j] = *reinterpret_cast<const uint32_t*>(base + oWS + j * 256 + lane * 4);
      }
    };
    auto arrive = [&](int64_t kt) {
      const int64_t ahead = nkt - 1 - kt;
      wait_stage<kOps, D>((int)(ahead < D - 2 ? ahead : D - 2));
      wait_lgkmcnt0();
      block_sync();
      if (kt + D - 1 < nkt) issue(kt + D - 1, (int)((kt + D - 1) % D));
    };

    auto kloop = [&](auto fullc) {
      constexpr bool FULL = decltype(fullc)::value;
      // Waves without rows (a short last M tile) run the same instruction stream on harmless data and
      // skip the epilogue: keeping the loop free of divergent branches lets the compiler wait for exactly
      // the LDS reads each MFMA needs instead of draining all of them.
      Frag cur, nxt;
      arrive(0);
      load_frag(0, cur);
      for (int64_t grp = 0; grp < g.ngrp2; grp++) {
        auto step = [&](auto jc) {
          constexpr int J = decltype(jc)::value;
          const int64_t kt = grp * 4 + J;
          const bool more = kt + 1 < nkt;
          auto mfmas = [&]() {
          {
            i32x8_t at[kTerms];
            at[0] = i32x8_t{(int)cur.x[0][0], (int)cur.x[0][1], (int)cur.x[0][2], (int)cur.x[0][3], (int)cur.x[1][0],
                            (int)cur.x[1][1], 0, 0};
            at[1] = i32x8_t{(int)cur.x[1][2], (int)cur.x[1][3], (int)cur.x[2][0], (int)cur.x[2][1], (int)cur.x[2][2],
                            (int)cur.x[2][3], 0, 0};
            at[2] = i32x8_t{(int)cur.x[3][0], (int)cur.x[3][1], (int)cur.x[3][2], (int)cur.x[3][3], (int)cur.x[4][0],
                            (int)cur.x[4][1], 0, 0};
#pragma unroll
            for (int t = 0; t < kTerms; t++)
#pragma unroll
              for (int j = 0; j < NB; j++)
                if (FULL || nt0 + j < g.nht)
                  acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(at[t], fp4_operand(cur.b[j]), acc[j], kFp6, kFp4, J,
                                                                           cur.sa[t], J, cur.sb[j]);
          }
          };
          if (more) {
            arrive(kt + 1);
            load_frag(kt + 1, nxt);
            mfmas();
            cur = nxt;
          } else {
            mfmas();
          }
        };
        step(std::integral_constant<int, 0>{});
        if (grp * 4 + 1 < nkt) step(std::integral_constant<int, 1>{});
        if (grp * 4 + 2 < nkt) step(std::integral_constant<int, 2>{});
        if (grp * 4 + 3 < nkt) step(std::integral_constant<int, 3>{});
      }
    };
    if (nt0 + NB <= g.nht) kloop(std::true_type{});
    else kloop(std::false_type{});

    if (valid) {
      const int h = lane >> 5;
#pragma unroll
      for (int j = 0; j < NB; j++) {
        if (nt0 + j >= g.nht) continue;
        const int64_t col = (nt0 + j) * 32 + (lane & 31);
        const float bias = b2 ? bf16_bits_to_f32(b2[(int64_t)e * g.H + col]) : 0.f;
#pragma unroll
        for (int q = 0; q < 16; q++) {
          const int rr = wave * 32 + 8 * (q >> 2) + 4 * h + (q & 3);
          const int pair = s_pair[rr];
          if (pair >= 0) obuf[(int64_t)pair * g.H + col] = s_w[rr] * (acc[j][q] + bias);
        }
      }
    }
  }
}

// y[t] = sum_j o_buf[t*k + j], fp32 sum in j order, bf16 out; eight columns per thread.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ obuf, uint16_t* __restrict__ y,
                                                      int64_t H8, int k, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / H8, c = i - t * H8;
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    const f32x4_t* src = reinterpret_cast<const f32x4_t*>(obuf) + ((t * k) * H8 + c) * 2;
    for (int j = 0; j < k; j++) {
      s0 += src[j * H8 * 2];
      s1 += src[j * H8 * 2 + 1];
    }
    u32x4_t o;
    o[0] = f32_to_bf16_bits(s0[0]) | (f32_to_bf16_bits(s0[1]) << 16);
    o[1] = f32_to_bf16_bits(s0[2]) | (f32_to_bf16_bits(s0[3]) << 16);
    o[2] = f32_to_bf16_bits(s1[0]) | (f32_to_bf16_bits(s1[1]) << 16);
    o[3] = f32_to_bf16_bits(s1[2]) | (f32_to_bf16_bits(s1[3]) << 16);
    reinterpret_cast<u32x4_t*>(y)[i] = o;
  }
}


}  // namespace

static unsigned tiles_grid_y(int64_t max_tiles) { return (unsigned)(max_tiles < 65535 ? max_tiles : 65535); }

// 1-D grid of the row-split kernels: every (tile, column block) item, rounded up to whole XCD rounds.
static unsigned rows_grid(int64_t max_tiles, int64_t nx) { return (unsigned)(kXcds * cdiv(max_tiles * nx, kXcds)); }

constexpr int kNW = 4;    // waves per workgroup of the column-split kernels (single row group tiles)
constexpr int kNACT = 4;  // activation tiles per workgroup of the row-split first GEMM
constexpr int kNB = 8;    // column tiles per workgroup of the row-split second GEMM

int launch_gemm1(int MT, const MoeGeom& g, const uint8_t* blob, const BlobOffsets& o, bool bias, const uint8_t* xq,
                 const uint8_t* xs, const int32_t* prow_pair, const void* tiles, const int32_t* ntiles, int64_t max_tiles,
                 uint8_t* actq, uint8_t* acts, int k, hipStream_t stream) {
  const uint16_t* b13 = bias ? (const uint16_t*)(blob + o.b13) : nullptr;
  const uint8_t* wq = blob + o.w13q;
  const uint32_t* ws = (const uint32_t*)(blob + o.w13s);
  const int4* tl = (const int4*)tiles;
  const unsigned gy = tiles_grid_y(max_tiles);
  switch (MT) {
    case 1:
      hipLaunchKernelGGL((gemm1_kernel<1, kNW, true>), dim3((unsigned)cdiv(g.nit, kNW), gy), dim3(kNW * 64), 0, stream,
                         wq, ws, b13, xq, xs, prow_pair, tl, ntiles, actq, acts, g, k);
      break;
    case 2:
      hipLaunchKernelGGL((gemm1_rows_kernel<2, kNACT, 4>), dim3(rows_grid(max_tiles, cdiv(g.nit, kNACT))), dim3(2 * 64), 0, stream,
                         wq, ws, b13, xq, xs, prow_pair, tl, ntiles, actq, acts, g, k);
      break;
    case 4:
      hipLaunchKernelGGL((gemm1_rows_kernel<4, kNACT, 4>), dim3(rows_grid(max_tiles, cdiv(g.nit, kNACT))), dim3(4 * 64), 0, stream,
                         wq, ws, b13, xq, xs, prow_pair, tl, ntiles, actq, acts, g, k);
      break;
    default:
      return MXFP4_ERR_SHAPE;
  }
  return hipGetLastError() == hipSuccess ? MXFP4_OK : MXFP4_ERR_DEVICE;
}

int launch_gemm2(int MT, const MoeGeom& g, const uint8_t* blob, const BlobOffsets& o, bool bias, const uint8_t* actq,
                 const uint8_t* acts, const int32_t* prow_pair, const float* topw, const void* tiles,
                 const int32_t* ntiles, int64_t max_tiles, float* obuf, int64_t T, int k, hipStream_t stream) {
  (void)T;
  const uint16_t* b2 = bias ? (const uint16_t*)(blob + o.b2) : nullptr;
  const uint8_t* wq = blob + o.w2q;
  const uint32_t* ws = (const uint32_t*)(blob + o.w2s);
  const int4* tl = (const int4*)tiles;
  const unsigned gy = tiles_grid_y(max_tiles);
  switch (MT) {
    case 1:
      hipLaunchKernelGGL((gemm2_kernel<1, kNW, true>), dim3((unsigned)cdiv(g.nht, kNW), gy), dim3(kNW * 64), 0, stream,
                         wq, ws, b2, actq, acts, prow_pair, topw, tl, ntiles, obuf, g, k);
      break;
    case 2:
      hipLaunchKernelGGL((gemm2_rows_kernel<2, kNB, 4>), dim3(rows_grid(max_tiles, cdiv(g.nht, kNB))), dim3(2 * 64), 0, stream,
                         wq, ws, b2, actq, acts, prow_pair, topw, tl, ntiles, obuf, g, k);
      break;
    case 4:
      hipLaunchKernelGGL((gemm2_rows_kernel<4, kNB, 4>), dim3(rows_grid(max_tiles, cdiv(g.nht, kNB))), dim3(4 * 64), 0, stream,
                         wq, ws, b2, actq, acts, prow_pair, topw, tl, ntiles, obuf, g, k);
      break;
    default:
      return MXFP4_ERR_SHAPE;
  }
  return hipGetLastError() == hipSuccess ? MXFP4_OK : MXFP4_ERR_DEVICE;
}

int launch_combine(const float* obuf, void* y, int64_t T, int64_t H, int k, hipStream_t stream) {
  const int64_t n = T * (H / 8);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (n > 0)
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, obuf, (uint16_t*)y, H / 8, k, n);
  return hipGetLastError() == hipSuccess ? MXFP4_OK : MXFP4_ERR_DEVICE;
}
