// Grouped expert GEMMs of the MoE layer on gfx950 block-scaled MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4), with the SwiGLU and the weighted scatter-combine fused into
// their epilogues.
//
// [NS: grouped w13 GEMM, SwiGLU = silu(w1 half) * (w3 half), grouped w2 GEMM, weighted top-k combine;
//  MXFP4 weights with E8M0 scales per 32 elements; P1 Implementation breakdown: the mixed-input fused
//  MoE multiplies packed 4-bit weights with per-32 group scales by 16-bit activations]
//
// The MFMA has no bf16 operand, so a bf16 activation enters as two E2M3 (FP6) terms x = hi + lo, each
// with its own E8M0 scale per 32 elements, and every product is issued twice (hi, lo) against the
// same FP4 weight registers.  FP6 x FP4 runs at the FP4 rate on gfx950.
//
// First GEMM, transposed: D[n][m] = sum_k W13[n][k] x[m][k], weights as the A operand (rows n = 32
// gate or up rows of one 32-column tile), tokens as the B operand (columns m = 32 tokens gathered from
// the sorted pair list).  Lane l of the 32x32 result holds token l%32 and rows 8*jj + 4*(l/32) + i, so
// gate and up of one column sit in the same lane (SwiGLU in registers) and a 32-element block of the
// activation is split over the two lane halves (one exchange for the block maximum).
//
// Second GEMM, not transposed: D[m][n] = sum_k act[m][k] W2[n][k]; lane l holds output column l%32 and
// rows 8*jj + 4*(l/32) + i, so each fp32 atomic instruction adds 2 x 32 consecutive floats.
#include "common.h"

namespace {

typedef decltype(__builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(bf16x32_t{}, 1.0f)) fp6x32_t;

MX_DEV u32x4_t ld16(const uint8_t* p) { return *reinterpret_cast<const u32x4_t*>(p); }

MX_DEV i32x8_t fp4_operand(u32x4_t v) {
  return i32x8_t{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
}
// 48 bytes = hi (6 dwords) then lo (6 dwords)
MX_DEV void fp6_pair_operands(const uint8_t* p, i32x8_t& hi, i32x8_t& lo) {
  const u32x4_t a = ld16(p), b = ld16(p + 16), c = ld16(p + 32);
  hi = i32x8_t{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], 0, 0};
  lo = i32x8_t{(int)b[2], (int)b[3], (int)c[0], (int)c[1], (int)c[2], (int)c[3], 0, 0};
}

constexpr int kFp4 = 4, kFp6 = 2;  // MFMA operand format codes (E2M1, E2M3)

// ------------------------------------------------------------------------------------------------
// First GEMM + SwiGLU + hi/lo split of the activation.
// grid: x = groups of 4 column tiles (one per wave), y = M tiles (tile list from the router).
template <int MT>
struct G1Acc {
  f32x16_t g[MT], u[MT];
};

template <int J, int MT>
MX_DEV void g1_ktile(G1Acc<MT>& acc, const uint8_t* wa, const uint8_t* const* xrow, int64_t kt, uint32_t sg, uint32_t su,
                     const uint32_t* sxh, const uint32_t* sxl, int nvalid_groups) {
  const i32x8_t ag = fp4_operand(ld16(wa + kt * 2048));
  const i32x8_t au = fp4_operand(ld16(wa + kt * 2048 + 1024));
#pragma unroll
  for (int mt = 0; mt < MT; mt++) {
    if (mt < nvalid_groups) {
      i32x8_t bh, bl;
      fp6_pair_operands(xrow[mt] + kt * 96, bh, bl);
      acc.g[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ag, bh, acc.g[mt], kFp4, kFp6, J, sg, J, sxh[mt]);
      acc.g[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ag, bl, acc.g[mt], kFp4, kFp6, J, sg, J, sxl[mt]);
      acc.u[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(au, bh, acc.u[mt], kFp4, kFp6, J, su, J, sxh[mt]);
      acc.u[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(au, bl, acc.u[mt], kFp4, kFp6, J, su, J, sxl[mt]);
    }
  }
}

MX_DEV float silu(float g) { return g / (1.0f + __expf(-g)); }

template <int MT>
__global__ __launch_bounds__(256) void gemm1_kernel(const uint8_t* __restrict__ w13q, const uint32_t* __restrict__ w13s,
                                                    const uint16_t* __restrict__ b13, const uint8_t* __restrict__ xq,
                                                    const uint8_t* __restrict__ xs, const int32_t* __restrict__ prow_pair,
                                                    const int4* __restrict__ tiles, const int32_t* __restrict__ ntiles,
                                                    uint8_t* __restrict__ actq, uint8_t* __restrict__ acts, MoeGeom g,
                                                    int k) {
  const int nt_all = *ntiles;
  for (int tile = blockIdx.y; tile < nt_all; tile += gridDim.y) {
  const int4 td = tiles[tile];
  const int e = td.x, prow0 = td.y, nrows = td.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t it = (int64_t)blockIdx.x * 4 + wave;
  if (it >= g.nit) return;  // wave-uniform and the same for every tile; the kernel has no barrier
  const int nvalid_groups = (nrows + 31) >> 5;
  const int64_t nblk1 = 2 * g.nkt1;

  const uint8_t* xrow[MT];
  const uint8_t* xsrow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; mt++) {
    const int r = mt * 32 + (lane & 31);
    int tok = 0;
    if (r < nrows) {
      const int pair = prow_pair[prow0 + r];
      if (pair >= 0) tok = pair / k;
    }
    xrow[mt] = xq + ((int64_t)tok * nblk1 + (lane >> 5)) * 48;
    xsrow[mt] = xs + (int64_t)tok * g.ngrp1 * 16 + (lane >> 5) * 4;
  }
  const uint8_t* wa = w13q + ((int64_t)e * g.nit + it) * g.nkt1 * 2048 + lane * 16;
  const uint32_t* wsa = w13s + ((int64_t)e * g.nit + it) * g.ngrp1 * 128 + lane;

  G1Acc<MT> acc;
#pragma unroll
  for (int mt = 0; mt < MT; mt++)
#pragma unroll
    for (int i = 0; i < 16; i++) { acc.g[mt][i] = 0.f; acc.u[mt][i] = 0.f; }

  for (int64_t grp = 0; grp < g.ngrp1; grp++) {
    const uint32_t sg = wsa[grp * 128], su = wsa[grp * 128 + 64];
    uint32_t sxh[MT], sxl[MT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      sxh[mt] = *reinterpret_cast<const uint32_t*>(xsrow[mt] + grp * 16);
      sxl[mt] = *reinterpret_cast<const uint32_t*>(xsrow[mt] + grp * 16 + 8);
    }
    const int64_t kt0 = grp * 4;
    g1_ktile<0, MT>(acc, wa, xrow, kt0, sg, su, sxh, sxl, nvalid_groups);
    if (kt0 + 1 < g.nkt1) g1_ktile<1, MT>(acc, wa, xrow, kt0 + 1, sg, su, sxh, sxl, nvalid_groups);
    if (kt0 + 2 < g.nkt1) g1_ktile<2, MT>(acc, wa, xrow, kt0 + 2, sg, su, sxh, sxl, nvalid_groups);
    if (kt0 + 3 < g.nkt1) g1_ktile<3, MT>(acc, wa, xrow, kt0 + 3, sg, su, sxh, sxl, nvalid_groups);
  }

  // ---- epilogue: bias, SwiGLU, bf16, hi/lo E2M3 split, store in the second GEMM's operand layout
  const int m = lane & 31, h = lane >> 5;
  float b1[16], b3[16];
#pragma unroll
  for (int q = 0; q < 16; q++) {
    const int n = 8 * (q >> 2) + 4 * h + (q & 3);
    if (b13) {
      b1[q] = bf16_bits_to_f32(b13[(int64_t)e * 2 * g.I + it * 32 + n]);
      b3[q] = bf16_bits_to_f32(b13[(int64_t)e * 2 * g.I + g.I + it * 32 + n]);
    } else {
      b1[q] = 0.f;
      b3[q] = 0.f;
    }
  }
  const int64_t kt2 = it >> 1, kb = it & 1;
  const bool pad_block = (it == g.nit - 1) && (g.nit & 1);  // the zero block that completes the last K tile
#pragma unroll
  for (int mt = 0; mt < MT; mt++) {
    if (mt >= nvalid_groups) continue;
    uint32_t ab[16];
    uint32_t amax = 0;
#pragma unroll
    for (int q = 0; q < 16; q++) {
      const float gv = acc.g[mt][q] + b1[q];
      const float uv = acc.u[mt][q] + b3[q];
      ab[q] = f32_to_bf16_bits(silu(gv) * uv);
      amax = max(amax, ab[q] & 0x7FFFu);
    }
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 32));
    const uint32_t ehi = e8m0_from_amax_bits(amax << 16);
    const float shi = e8m0_as_scale_operand(ehi);
    bf16x32_t v;
#pragma unroll
    for (int q = 0; q < 16; q++) {
      v[q] = __builtin_bit_cast(__bf16, (uint16_t)ab[q]);
      v[16 + q] = __builtin_bit_cast(__bf16, (uint16_t)0);
    }
    const fp6x32_t hi = __builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(v, shi);
    const auto deq = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(hi, shi);
    uint32_t rmax = 0;
#pragma unroll
    for (int q = 0; q < 16; q++) {
      const uint32_t rb = f32_to_bf16_bits(bf16_bits_to_f32(ab[q]) - deq[q]);
      v[q] = __builtin_bit_cast(__bf16, (uint16_t)rb);
      rmax = max(rmax, rb & 0x7FFFu);
    }
    rmax = max(rmax, (uint32_t)__shfl_xor((int)rmax, 32));
    const uint32_t elo = e8m0_from_amax_bits(rmax << 16);
    const fp6x32_t lo = __builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(v, e8m0_as_scale_operand(elo));

    const int64_t rg = (prow0 >> 5) + mt;
    uint8_t* chunk = actq + ((rg * g.nkt2 + kt2) * 64 + kb * 32 + m) * 48;
    uint32_t* hp = reinterpret_cast<uint32_t*>(chunk + h * 12);
    hp[0] = hi[0]; hp[1] = hi[1]; hp[2] = hi[2];
    uint32_t* lp = reinterpret_cast<uint32_t*>(chunk + 24 + h * 12);
    lp[0] = lo[0]; lp[1] = lo[1]; lp[2] = lo[2];
    uint8_t* sc = acts + ((rg * g.ngrp2 + (kt2 >> 2)) * 64 + kb * 32 + m) * 8 + (kt2 & 3);
    sc[h * 4] = (uint8_t)(h == 0 ? ehi : elo);
    if (pad_block) {
      uint32_t* zp = reinterpret_cast<uint32_t*>(actq + ((rg * g.nkt2 + kt2) * 64 + 32 + m) * 48 + h * 24);
#pragma unroll
      for (int q = 0; q < 6; q++) zp[q] = 0;
      acts[((rg * g.ngrp2 + (kt2 >> 2)) * 64 + 32 + m) * 8 + (kt2 & 3) + h * 4] = 0;
    }
  }
  }
}

// ------------------------------------------------------------------------------------------------
// Second GEMM + bias + routing weight + fp32 atomic combine.
// grid: x = groups of 4 column tiles of H (one per wave), y = M tiles.
template <int J, int MT>
MX_DEV void g2_ktile(f32x16_t* acc, const uint8_t* wb, const uint8_t* const* arow, int64_t kt, uint32_t sb,
                     const uint32_t* sah, const uint32_t* sal, int nvalid_groups) {
  const i32x8_t b = fp4_operand(ld16(wb + kt * 1024));
#pragma unroll
  for (int mt = 0; mt < MT; mt++) {
    if (mt < nvalid_groups) {
      i32x8_t ah, al;
      fp6_pair_operands(arow[mt] + kt * 3072, ah, al);
      acc[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ah, b, acc[mt], kFp6, kFp4, J, sah[mt], J, sb);
      acc[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(al, b, acc[mt], kFp6, kFp4, J, sal[mt], J, sb);
    }
  }
}

template <int MT>
__global__ __launch_bounds__(256) void gemm2_kernel(const uint8_t* __restrict__ w2q, const uint32_t* __restrict__ w2s,
                                                    const uint16_t* __restrict__ b2, const uint8_t* __restrict__ actq,
                                                    const uint8_t* __restrict__ acts, const int32_t* __restrict__ prow_pair,
                                                    const float* __restrict__ topw, const int4* __restrict__ tiles,
                                                    const int32_t* __restrict__ ntiles, float* __restrict__ yacc,
                                                    MoeGeom g, int k) {
  const int nt_all = *ntiles;
  for (int tile = blockIdx.y; tile < nt_all; tile += gridDim.y) {
  const int4 td = tiles[tile];
  const int e = td.x, prow0 = td.y, nrows = td.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nt = (int64_t)blockIdx.x * 4 + wave;
  if (nt >= g.nht) return;  // wave-uniform and the same for every tile
  const int nvalid_groups = (nrows + 31) >> 5;

  const uint8_t* arow[MT];
  const uint8_t* sarow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; mt++) {
    const int64_t rg = (prow0 >> 5) + mt;
    arow[mt] = actq + (rg * g.nkt2 * 64 + lane) * 48;
    sarow[mt] = acts + (rg * g.ngrp2 * 64 + lane) * 8;
  }
  const uint8_t* wb = w2q + ((int64_t)e * g.nht + nt) * g.nkt2 * 1024 + lane * 16;
  const uint32_t* wsb = w2s + ((int64_t)e * g.nht + nt) * g.ngrp2 * 64 + lane;

  f32x16_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; mt++)
#pragma unroll
    for (int i = 0; i < 16; i++) acc[mt][i] = 0.f;

  for (int64_t grp = 0; grp < g.ngrp2; grp++) {
    const uint32_t sb = wsb[grp * 64];
    uint32_t sah[MT], sal[MT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      const u32x2_t s = *reinterpret_cast<const u32x2_t*>(sarow[mt] + grp * 512);
      sah[mt] = s[0];
      sal[mt] = s[1];
    }
    const int64_t kt0 = grp * 4;
    g2_ktile<0, MT>(acc, wb, arow, kt0, sb, sah, sal, nvalid_groups);
    if (kt0 + 1 < g.nkt2) g2_ktile<1, MT>(acc, wb, arow, kt0 + 1, sb, sah, sal, nvalid_groups);
    if (kt0 + 2 < g.nkt2) g2_ktile<2, MT>(acc, wb, arow, kt0 + 2, sb, sah, sal, nvalid_groups);
    if (kt0 + 3 < g.nkt2) g2_ktile<3, MT>(acc, wb, arow, kt0 + 3, sb, sah, sal, nvalid_groups);
  }

  const int64_t col = nt * 32 + (lane & 31);
  const float bias = b2 ? bf16_bits_to_f32(b2[(int64_t)e * g.H + col]) : 0.f;
  const int h = lane >> 5;
#pragma unroll
  for (int mt = 0; mt < MT; mt++) {
    if (mt >= nvalid_groups) continue;
#pragma unroll
    for (int q = 0; q < 16; q++) {
      const int r = mt * 32 + 8 * (q >> 2) + 4 * h + (q & 3);
      if (r < nrows) {
        const int pair = prow_pair[prow0 + r];
        if (pair >= 0) {
          const int64_t t = pair / k;
          atomicAdd(&yacc[t * g.H + col], topw[pair] * (acc[mt][q] + bias));
        }
      }
    }
  }
  }
}

}  // namespace

static unsigned tiles_grid_y(int64_t max_tiles) { return (unsigned)(max_tiles < 65535 ? max_tiles : 65535); }

int launch_gemm1(int MT, const MoeGeom& g, const uint8_t* blob, const BlobOffsets& o, bool bias, const uint8_t* xq,
                 const uint8_t* xs, const int32_t* prow_pair, const void* tiles, const int32_t* ntiles, int64_t max_tiles,
                 uint8_t* actq, uint8_t* acts, int k, hipStream_t stream) {
  const uint16_t* b13 = bias ? (const uint16_t*)(blob + o.b13) : nullptr;
  dim3 grid((unsigned)cdiv(g.nit, 4), tiles_grid_y(max_tiles));
#define G1(MTV)                                                                                                   \
  hipLaunchKernelGGL(gemm1_kernel<MTV>, grid, dim3(256), 0, stream, blob + o.w13q, (const uint32_t*)(blob + o.w13s), \
                     b13, xq, xs, prow_pair, (const int4*)tiles, ntiles, actq, acts, g, k)
  switch (MT) {
    case 1: G1(1); break;
    case 2: G1(2); break;
    case 4: G1(4); break;
    default: return MXFP4_ERR_SHAPE;
  }
#undef G1
  return hipGetLastError() == hipSuccess ? MXFP4_OK : MXFP4_ERR_DEVICE;
}

int launch_gemm2(int MT, const MoeGeom& g, const uint8_t* blob, const BlobOffsets& o, bool bias, const uint8_t* actq,
                 const uint8_t* acts, const int32_t* prow_pair, const float* topw, const void* tiles,
                 const int32_t* ntiles, int64_t max_tiles, float* yacc, int k, hipStream_t stream) {
  const uint16_t* b2 = bias ? (const uint16_t*)(blob + o.b2) : nullptr;
  dim3 grid((unsigned)cdiv(g.nht, 4), tiles_grid_y(max_tiles));
#define G2(MTV)                                                                                                   \
  hipLaunchKernelGGL(gemm2_kernel<MTV>, grid, dim3(256), 0, stream, blob + o.w2q, (const uint32_t*)(blob + o.w2s), b2, \
                     actq, acts, prow_pair, topw, (const int4*)tiles, ntiles, yacc, g, k)
  switch (MT) {
    case 1: G2(1); break;
    case 2: G2(2); break;
    case 4: G2(4); break;
    default: return MXFP4_ERR_SHAPE;
  }
#undef G2
  return hipGetLastError() == hipSuccess ? MXFP4_OK : MXFP4_ERR_DEVICE;
}
