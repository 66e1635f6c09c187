// MoE front and back: activation preparation, top-k routing, the stable counting sort of
// (token, expert) pairs with the GEMM tile schedule, and the final fp32 -> bf16 combine output.
//
// [NS: top-k routing of softmax(router logits) renormalized over the selected experts; the router
//  sort/permute/gather step; the weighted top-k combine]
#include "common.h"

namespace {

#define GRID_STRIDE(i, n) for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (n); i += (int64_t)gridDim.x * blockDim.x)

typedef decltype(__builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(bf16x32_t{}, 1.0f)) fp6x32_t;

// Split 32 bf16 values into kTerms E2M3 terms x = t0 + t1 + t2: each term is the current remainder
// quantized with its own E8M0 scale from the 0.75 round-up rule (block maximum / scale < 7 <= 7.5, the
// E2M3 maximum, so no term saturates), and the next remainder is exact in bf16 (a term is a multiple
// of the remainder's ulp within one grid step of it).
struct Fp6Split {
  fp6x32_t t[kTerms];
  uint32_t e[kTerms];
};

MX_DEV uint32_t amax_bits32(const uint32_t* w) {  // 16 words = 32 bf16 -> largest magnitude bits
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 16; i++) m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  return m;
}

MX_DEV Fp6Split split_fp6(const uint32_t* w /* 16 words */) {
  Fp6Split p;
  uint32_t cur[16];
#pragma unroll
  for (int i = 0; i < 16; i++) cur[i] = w[i];
#pragma unroll
  for (int term = 0; term < kTerms; term++) {
    bf16x32_t v;
#pragma unroll
    for (int i = 0; i < 16; i++) {
      bf16x2_t two = __builtin_bit_cast(bf16x2_t, cur[i]);
      v[2 * i] = two[0];
      v[2 * i + 1] = two[1];
    }
    p.e[term] = e8m0_from_amax_bits(amax_bits32(cur) << 16);
    const float sc = e8m0_as_scale_operand(p.e[term]);
    p.t[term] = __builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(v, sc);
    if (term + 1 < kTerms) {
      const auto deq = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(p.t[term], sc);
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const float a = bf16_bits_to_f32(cur[i] & 0xFFFFu) - deq[2 * i];
        const float b = bf16_bits_to_f32(cur[i] >> 16) - deq[2 * i + 1];
        cur[i] = f32_to_bf16_bits(a) | (f32_to_bf16_bits(b) << 16);
      }
    }
  }
  return p;
}

// x [T, ldx] bf16 -> xq/xs (three E2M3 terms per 32-element block, K padded to a multiple of 64 with
// zero blocks); also clears the per-expert pair counters.
__global__ __launch_bounds__(256) void xprep_kernel(const uint16_t* __restrict__ x, int64_t ldx, int64_t H, int64_t nblk,
                                                    int64_t ngrp, uint8_t* __restrict__ xq, uint8_t* __restrict__ xs,
                                                    int32_t* __restrict__ counts, int E,
                                                    int64_t n) {
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < E; i += blockDim.x) counts[i] = 0;
  GRID_STRIDE(i, n) {
    const int64_t t = i / nblk, b = i % nblk;
    uint32_t w[16];
    const bool in = b < H / 32;
    if (in) {
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + t * ldx + b * 32);
#pragma unroll
      for (int j = 0; j < 4; j++) {
        u32x4_t v = src[j];
        w[4 * j] = v[0]; w[4 * j + 1] = v[1]; w[4 * j + 2] = v[2]; w[4 * j + 3] = v[3];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; j++) w[j] = 0;
    }
    const Fp6Split p = split_fp6(w);
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(xq + (t * nblk + b) * kSlot);
    dst[0] = u32x4_t{p.t[0][0], p.t[0][1], p.t[0][2], p.t[0][3]};
    dst[1] = u32x4_t{p.t[0][4], p.t[0][5], p.t[1][0], p.t[1][1]};
    dst[2] = u32x4_t{p.t[1][2], p.t[1][3], p.t[1][4], p.t[1][5]};
    dst[3] = u32x4_t{p.t[2][0], p.t[2][1], p.t[2][2], p.t[2][3]};
    dst[4] = u32x4_t{p.t[2][4], p.t[2][5], 0u, 0u};
    const int64_t grp = b >> 3, j = (b & 7) >> 1, par = b & 1;
    uint8_t* s = xs + (t * ngrp + grp) * (kTerms * 8) + par * 4 + j;
#pragma unroll
    for (int term = 0; term < kTerms; term++) s[term * 8] = (uint8_t)p.e[term];
  }
}

// Order-preserving key of an fp32 logit with -0.0 folded onto +0.0; larger key = larger logit.
MX_DEV uint32_t logit_key(float l) {
  uint32_t u = __float_as_uint(l);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kMaxPerLane = 16;  // E <= 1024

// One wave per token: k rounds of a wave-wide arg-max over 64-bit keys (logit key, inverted expert
// index), so equal logits go to the lower expert index; softmax weights of the selected experts.
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int64_t T, int E, int k,
                                                    int renormalize, int32_t* __restrict__ ids, float* __restrict__ wts,
                                                    int32_t* __restrict__ counts) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave
  const float* lt = logits + t * E;
  uint64_t key[kMaxPerLane];
  float val[kMaxPerLane];
#pragma unroll
  for (int j = 0; j < kMaxPerLane; j++) {
    const int idx = lane + 64 * j;
    if (idx < E) {
      val[j] = lt[idx];
      key[j] = ((uint64_t)logit_key(val[j]) << 32) | (uint32_t)(~idx);
    } else {
      val[j] = 0.f;
      key[j] = 0;
    }
  }
  int my_id = 0;
  float my_l = 0.f, lmax = 0.f;
  for (int r = 0; r < k; r++) {
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < kMaxPerLane; j++) best = key[j] > best ? key[j] : best;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)best, off);
      const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(best >> 32), off);
      const uint64_t o = ((uint64_t)hi << 32) | lo;
      best = o > best ? o : best;
    }
    const int id = (int)(~(uint32_t)best);
    // owner lane clears the winner and broadcasts its logit
    float wl = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxPerLane; j++) {
      if (lane + 64 * j == id) {
        wl = val[j];
        key[j] = 0;
      }
    }
    wl = __shfl(wl, id & 63);
    if (r == 0) lmax = wl;
    if (lane == r) {
      my_id = id;
      my_l = wl;
    }
  }
  const float ex = lane < k ? __expf(my_l - lmax) : 0.f;
  float den = 0.f;
  if (renormalize) {
    den = ex;
  } else {
#pragma unroll
    for (int j = 0; j < kMaxPerLane; j++)
      if (lane + 64 * j < E) den += __expf(val[j] - lmax);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off);
  if (lane < k) {
    ids[t * k + lane] = my_id;
    wts[t * k + lane] = ex / den;
    atomicAdd(&counts[my_id], 1);
  }
}

// One workgroup per expert: prefix sums of the counts of lower experts (compact and padded offsets,
// M-tile offset), the tile list of this expert, and a stable scatter of its pairs in token order.
__global__ __launch_bounds__(256) void place_kernel(const int32_t* __restrict__ ids, const int32_t* __restrict__ counts,
                                                    int64_t T, int k, int E, int BM, int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ poffsets, int32_t* __restrict__ sorted_pairs,
                                                    int32_t* __restrict__ prow_pair, int4* __restrict__ tiles,
                                                    int32_t* __restrict__ ntiles) {
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ int red[4][3];
  __shared__ int wsum[4];
  int s0 = 0, s1 = 0, s2 = 0;
  for (int i = tid; i < e; i += 256) {
    const int c = counts[i];
    s0 += c;
    s1 += (c + 31) & ~31;
    s2 += (c + BM - 1) / BM;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    s0 += __shfl_xor(s0, off);
    s1 += __shfl_xor(s1, off);
    s2 += __shfl_xor(s2, off);
  }
  if (lane == 0) { red[wave][0] = s0; red[wave][1] = s1; red[wave][2] = s2; }
  __syncthreads();
  const int off = red[0][0] + red[1][0] + red[2][0] + red[3][0];
  const int poff = red[0][1] + red[1][1] + red[2][1] + red[3][1];
  const int toff = red[0][2] + red[1][2] + red[2][2] + red[3][2];
  const int n = counts[e];
  const int npad = (n + 31) & ~31;
  const int nt = (n + BM - 1) / BM;
  if (tid == 0) {
    offsets[e] = off;
    poffsets[e] = poff;
    if (e == E - 1) {
      offsets[E] = off + n;
      poffsets[E] = poff + npad;
      *ntiles = toff + nt;
    }
  }
  for (int i = tid; i < nt; i += 256) tiles[toff + i] = make_int4(e, poff + i * BM, min(BM, n - i * BM), 0);
  for (int i = n + tid; i < npad; i += 256) prow_pair[poff + i] = -1;
  if (n == 0) return;
  int base = 0;
  for (int64_t t0 = 0; t0 < T; t0 += 256) {
    const int64_t t = t0 + tid;
    int j = -1;
    if (t < T)
      for (int jj = 0; jj < k; jj++)
        if (ids[t * k + jj] == e) j = jj;
    const bool f = j >= 0;
    const uint64_t bal = __ballot(f);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    __syncthreads();
    if (lane == 0) wsum[wave] = __popcll(bal);
    __syncthreads();
    int wbase = 0;
    for (int q = 0; q < wave; q++) wbase += wsum[q];
    const int total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    if (f) {
      const int pos = base + wbase + before;
      const int32_t pair = (int32_t)(t * k + j);
      sorted_pairs[off + pos] = pair;
      prow_pair[poff + pos] = pair;
    }
    base += total;
    if (base >= n) break;  // uniform: every thread sees the same total
  }
}

inline unsigned grid_for(int64_t n, int threads = 256) {
  int64_t b = (n + threads - 1) / threads;
  if (b > 65536) b = 65536;
  if (b < 1) b = 1;
  return (unsigned)b;
}

}  // namespace

int launch_xprep(const void* x, int64_t T, int64_t ldx, const MoeGeom& g, void* xq, void* xs, int32_t* counts,
                 hipStream_t stream) {
  const int64_t nblk = 2 * g.nkt1;
  const int64_t n = T * nblk;
  hipLaunchKernelGGL(xprep_kernel, dim3(grid_for(n)), dim3(256), 0, stream, (const uint16_t*)x, ldx, g.H, nblk,
                     g.ngrp1, (uint8_t*)xq, (uint8_t*)xs, counts, (int)g.E, n);
  return hipGetLastError() == hipSuccess ? MXFP4_OK : MXFP4_ERR_DEVICE;
}

__global__ void zero_i32_kernel(int32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

int launch_zero_i32(int32_t* p, int n, hipStream_t stream) {
  if (n > 0) hipLaunchKernelGGL(zero_i32_kernel, dim3(grid_for(n)), dim3(256), 0, stream, p, n);
  return hipGetLastError() == hipSuccess ? MXFP4_OK : MXFP4_ERR_DEVICE;
}

int launch_route(const float* logits, int64_t T, int E, int k, int renormalize, int32_t* ids, float* w,
                 int32_t* counts, hipStream_t stream) {
  if (T > 0)
    hipLaunchKernelGGL(route_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, stream, logits, T, E, k,
                       renormalize, ids, w, counts);
  return hipGetLastError() == hipSuccess ? MXFP4_OK : MXFP4_ERR_DEVICE;
}

int launch_place(const int32_t* ids, const int32_t* counts, int64_t T, int k, int E, int BM, int32_t* offsets,
                 int32_t* poffsets, int32_t* sorted_pairs, int32_t* prow_pair, void* tiles, int32_t* ntiles,
                 hipStream_t stream) {
  hipLaunchKernelGGL(place_kernel, dim3((unsigned)E), dim3(256), 0, stream, ids, counts, T, k, E, BM, offsets,
                     poffsets, sorted_pairs, prow_pair, (int4*)tiles, ntiles);
  return hipGetLastError() == hipSuccess ? MXFP4_OK : MXFP4_ERR_DEVICE;
}

