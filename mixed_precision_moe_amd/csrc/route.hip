// MoE front: activation preparation, top-k routing, and the stable counting sort of (token, expert)
// pairs that lays out the grouped GEMMs' rows and tile schedule.
//
// [DEF: top-k routing of softmax(router logits) renormalized over the selected experts; the router
//  sort/permute/gather step]
//
// The forward pass runs the front in two launches: front_kernel (the activation split and the routing
// side by side: the first workgroups route one block of kRouteTokens tokens each -- top-k per token,
// the block's expert histogram counted in LDS and written whole -- and the others split the
// activations) and place_kernel (per block of tokens: prefix sums over blocks and experts from the
// histograms, the block's pairs ranked per expert in token order and written to their rows; the first
// workgroup also writes the expert offsets, the padded row offsets, the M-tile lists and the padding
// rows).  The resulting order is stable: pairs of one expert appear in increasing token order.  The
// routing-only entry point launches the routing workgroups alone (route_kernel).
#include "common.h"
#include "internal.h"

namespace {

// x [T, ldx] bf16 -> xq: per 32-element block the terms of activation format AF (layout.h), each the
// current remainder quantized with its own E8M0 scale:
//   kActBf16: t0 = E2M3 of x, t1 = E2M3 of x - t0, t2 = E2M1 of x - t0 - t1, scales from the 0.75
//             round-up rule (an E2M3 term's maximum / scale < 7 <= 7.5, the E2M3 maximum, so it does
//             not saturate; the last term may, by at most 1/7 of its own maximum).  Each remainder of a
//             bf16 value after its rounding to a coarser grid is again exact in bf16.
//   kActMxfp8: one E4M3 term, scale rule for E4M3 (no saturation)
//   kActMxfp4: one E2M1 term, the weights' rule
// K is padded to a multiple of 64 with zero blocks.
//
// A wave handles 64 consecutive blocks (block gi = token * nblk + b), lane l computing block l.  Its
// global accesses are staged through LDS so that every load and store instruction covers 1 KB of
// consecutive bytes: 16-byte chunk c = 64 j + l of the wave's 4 KB of x is loaded by lane l in load j and
// written to LDS, lane l then reads its block's four chunks; lane l writes its slot and scale dword into
// record l / 2 (blocks 2r and 2r + 1 form the K-step record r), and the wave's 32 records (consecutive
// in xq) leave as 1 KB stores.  A wave takes the group indices wv0, wv0 + nw, ... below wv_end with its
// own LDS stage (max(4 KB, 32 records)): the records may overwrite the staged input, since every lane
// has read its x chunks (an earlier LDS instruction of the same wave) before any lane writes a record.
// The loads of a wave's next group are issued before the current group is converted and stored.
template <int AF>
MX_DEV void xprep_waves(const uint16_t* __restrict__ x, int64_t ldx, int64_t H, int64_t nblk, uint8_t* __restrict__ xq,
                        int64_t n, int64_t wv0, int64_t wv_end, int64_t nw, uint8_t* stage) {
  uint8_t* stage_in = stage;
  uint8_t* stage_out = stage;
  constexpr int SLOT = act_slot(AF), REC = act_rec(AF);
  const int lane = threadIdx.x & 63;
  const int64_t hb = H / 32;  // real blocks per token
  // coalesced loads of group wv: chunk c = 64 j + lane is part c % 4 of block c / 4.  The group's first
  // token comes from one (wave-uniform) division; every lane loads (a chunk past the data reads x's
  // first chunk, and its value is replaced by zero when it is staged), so each group is four loads.
  auto load = [&](int64_t wv, u32x4_t (&v)[4], uint32_t& okm) __attribute__((always_inline)) {
    const int64_t wu = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(wv >> 32)) << 32) |
                                 (uint32_t)__builtin_amdgcn_readfirstlane((int)wv));  // wv, in scalar registers
    const int64_t gb = wu * 64;  // the group's first block
    const int64_t t0 = gb / nblk;
    const int r0 = (int)(gb - t0 * nblk);
    okm = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int c = 64 * j + lane;
      const int loc = r0 + c / 4;          // block index from token t0's first block (< nblk + 64)
      const int dt = loc / (int)nblk;
      const int b = loc - dt * (int)nblk;
      const bool ok = gb + c / 4 < n && b < hb;
      okm |= ok ? 1u << j : 0u;
      const uint16_t* src = ok ? x + (t0 + dt) * ldx + b * 32 + (c % 4) * 8 : x;
      v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src));
    }
  };
  u32x4_t cur[4], nxt[4] = {};
  uint32_t okc = 0, okn = 0;
  if (wv0 < wv_end) load(wv0, cur, okc);
  for (int64_t wv = wv0; wv < wv_end; wv += nw) {
    const int64_t g0 = wv * 64;
    if (wv + nw < wv_end) load(wv + nw, nxt, okn);
#pragma unroll
    for (int j = 0; j < 4; j++)
      *reinterpret_cast<u32x4_t*>(&stage_in[(64 * j + lane) * 16]) = (okc >> j) & 1u ? cur[j] : u32x4_t{0u, 0u, 0u, 0u};
    __builtin_amdgcn_wave_barrier();  // the wave's LDS writes before its reads (single wave, in order)
    uint32_t w[16];
#pragma unroll
    for (int p = 0; p < 4; p++) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(&stage_in[lane * 64 + p * 16]);
      w[4 * p] = v[0]; w[4 * p + 1] = v[1]; w[4 * p + 2] = v[2]; w[4 * p + 3] = v[3];
    }
    uint32_t slot[SLOT / 4];
    uint32_t scales;
    if constexpr (AF == kActBf16) {
      scales = split3_bf16(w, slot);
    } else if constexpr (AF == kActMxfp8) {
      const uint32_t e = e8m0_e4m3_from_amax_bits(amax_bits32(w) << 16);
      fp8_from_bf16(w, e8m0_as_scale_operand(e), slot);
      scales = e;
    } else {
      const uint32_t e = e8m0_from_amax_bits(amax_bits32(w) << 16);
      fp4_from_bf16(w, e8m0_as_scale_operand(e), slot);
      scales = e;
    }
    uint8_t* rec = &stage_out[(lane >> 1) * REC];
    u32x4_t* sl = reinterpret_cast<u32x4_t*>(rec + (lane & 1) * SLOT);
    static_assert(SLOT % 16 == 0, "whole 16-byte stores");
#pragma unroll
    for (int d = 0; d < SLOT / 16; d++)
      sl[d] = u32x4_t{slot[4 * d], slot[4 * d + 1], slot[4 * d + 2], slot[4 * d + 3]};
    reinterpret_cast<uint32_t*>(rec + 2 * SLOT)[lane & 1] = scales;
    // the record's last 8 bytes: zero
    if (lane & 1) *reinterpret_cast<u32x2_t*>(rec + 2 * SLOT + 8) = u32x2_t{0u, 0u};
    __builtin_amdgcn_wave_barrier();
    // coalesced stores: 16-byte chunk c = 64 j + lane of the wave's 32 records (g0 is even, so the
    // wave's first record is g0 / 2; a record exists when its first block does)
    const int64_t r0 = g0 / 2;
#pragma unroll
    for (int j = 0; j < (2 * REC + 63) / 64; j++) {
      const int c = 64 * j + lane;
      if (c < 2 * REC && 2 * (r0 + (c * 16) / REC) < n)
        *reinterpret_cast<u32x4_t*>(xq + r0 * REC + c * 16) = *reinterpret_cast<const u32x4_t*>(&stage_out[c * 16]);
    }
    __builtin_amdgcn_wave_barrier();  // the next iteration's LDS writes after these reads
#pragma unroll
    for (int j = 0; j < 4; j++) cur[j] = nxt[j];
    okc = okn;
  }
}

// Order-preserving key of an fp32 logit with -0.0 folded onto +0.0; larger key = larger logit.
MX_DEV uint32_t logit_key(float l) {
  uint32_t u = __float_as_uint(l);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
MX_DEV float key_logit(uint32_t k) { return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k); }

// Wave-wide maximum, uniform result: DPP max inside each row of 16 lanes (xor 1, xor 2, rotate 4,
// rotate 8), then the four row maxima through scalar lane reads.
MX_DEV uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));  // row_ror:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));  // row_ror:8
  uint32_t r = 0;
#pragma unroll
  for (int row = 0; row < 4; row++) r = max(r, (uint32_t)__builtin_amdgcn_readlane((int)v, 16 * row));
  return r;
}
MX_DEV uint32_t wave_min_u32(uint32_t v) {
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));
  uint32_t r = 0xFFFFFFFFu;
#pragma unroll
  for (int row = 0; row < 4; row++) r = min(r, (uint32_t)__builtin_amdgcn_readlane((int)v, 16 * row));
  return r;
}
MX_DEV float wave_sum_f32(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
  float r = 0.f;
#pragma unroll
  for (int row = 0; row < 4; row++) r += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16 * row));
  return r;
}

// Routing of NT tokens by one wave, their selections interleaved (independent chains): k rounds of a
// wave-wide maximum of the logit keys, the winner being the lowest expert index holding that key (a
// wave-wide minimum over the indices of the lanes' slots that hold it), so equal logits go to the lower
// expert index; the winner's logit is read back from its key.  Softmax weights of the selected experts (renormalized over them, or over all experts).
// For token i, lane j < k returns pair j's expert and weight.  NPL logits per lane (E <= 64 * NPL).
template <int NPL, int NT>
MX_DEV void route_tokens(const float (&val)[NT][NPL], int E, int k, int renormalize, int (&my_id)[NT],
                         float (&my_w)[NT]) {
  const int lane = threadIdx.x & 63;
  uint32_t key[NT][NPL];  // 0 = absent or already selected (no logit maps to 0)
  float my_l[NT], lmax[NT];
#pragma unroll
  for (int i = 0; i < NT; i++) {
#pragma unroll
    for (int j = 0; j < NPL; j++) key[i][j] = lane + 64 * j < E ? logit_key(val[i][j]) : 0u;
    my_id[i] = 0;
    my_l[i] = 0.f;
    lmax[i] = 0.f;
  }
  for (int r = 0; r < k; r++) {
    uint32_t best[NT];
#pragma unroll
    for (int i = 0; i < NT; i++) {
      best[i] = 0;
#pragma unroll
      for (int j = 0; j < NPL; j++) best[i] = max(best[i], key[i][j]);
    }
#pragma unroll
    for (int i = 0; i < NT; i++) best[i] = wave_max_u32(best[i]);
    uint32_t cand[NT];
#pragma unroll
    for (int i = 0; i < NT; i++) {
      cand[i] = 0xFFFFFFFFu;
#pragma unroll
      for (int j = NPL - 1; j >= 0; j--)
        if (key[i][j] == best[i]) cand[i] = (uint32_t)(lane + 64 * j);
    }
#pragma unroll
    for (int i = 0; i < NT; i++) cand[i] = wave_min_u32(cand[i]);
#pragma unroll
    for (int i = 0; i < NT; i++) {
      const int id = (int)cand[i];
      const float wl = key_logit(best[i]);
#pragma unroll
      for (int j = 0; j < NPL; j++)
        if (lane + 64 * j == id) key[i][j] = 0;
      if (r == 0) lmax[i] = wl;
      if (lane == r) {
        my_id[i] = id;
        my_l[i] = wl;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NT; i++) {
    const float ex = lane < k ? __expf(my_l[i] - lmax[i]) : 0.f;
    float den;
    if (renormalize) {
      den = wave_sum_f32(ex);
    } else {
      float part = 0.f;
#pragma unroll
      for (int j = 0; j < NPL; j++)
        if (lane + 64 * j < E) part += __expf(val[i][j] - lmax[i]);
      den = wave_sum_f32(part);
    }
    my_w[i] = ex / den;
  }
}

// Reductions over each row of 16 lanes (DPP: quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_ror:4,
// row_ror:8); every lane of a row gets its row's result.
MX_DEV uint32_t row_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));
  return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));
}
MX_DEV uint32_t row_min_u32(uint32_t v) {
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));
  return min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));
}
MX_DEV float row_sum_f32(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
}

// Routing of four tokens per wave, one per row of 16 lanes (E <= 16 * NPR, k <= 16): the same
// selection as route_tokens with row-wide reductions -- lane q of a row holds experts q + 16 j, and the
// row minimum of the indices that hold the maximum gives the lowest one.  For the row's
// token, lane q < k returns pair q's expert and weight.
template <int NPR>
MX_DEV void route_rows(const float* val, int E, int k, int renormalize, int& my_id, float& my_w) {
  const int lane = threadIdx.x & 63, q = lane & 15;
  uint32_t key[NPR];
#pragma unroll
  for (int j = 0; j < NPR; j++) key[j] = q + 16 * j < E ? logit_key(val[j]) : 0u;
  my_id = 0;
  float my_l = 0.f, lmax = 0.f;
  for (int r = 0; r < k; r++) {
    uint32_t best = 0;
#pragma unroll
    for (int j = 0; j < NPR; j++) best = max(best, key[j]);
    best = row_max_u32(best);
    uint32_t cand = 0xFFFFFFFFu;
#pragma unroll
    for (int j = NPR - 1; j >= 0; j--)
      if (key[j] == best) cand = (uint32_t)(q + 16 * j);
    const int id = (int)row_min_u32(cand);
    const float wl = key_logit(best);
#pragma unroll
    for (int j = 0; j < NPR; j++)
      if (q + 16 * j == id) key[j] = 0;
    if (r == 0) lmax = wl;
    if (q == r) {
      my_id = id;
      my_l = wl;
    }
  }
  const float ex = q < k ? __expf(my_l - lmax) : 0.f;
  float den;
  if (renormalize) {
    den = row_sum_f32(ex);
  } else {
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < NPR; j++)
      if (q + 16 * j < E) part += __expf(val[j] - lmax);
    den = row_sum_f32(part);
  }
  my_w = ex / den;
}

// Routing of token block blk (kRouteTokens tokens) by one workgroup of 1024 threads: wave w takes tokens
// 4w .. 4w + 3 of the block -- one per row of 16 lanes up to 256 experts and top-16, else one after
// another across the wave with their selections interleaved (two at a time past 512 experts, for
// registers) -- and writes ids and weights.  Each pair is counted into the block's expert histogram
// in LDS and marks its token in the expert's 64-bit token mask; after a barrier each pair's rank among
// the block's pairs of its expert (the earlier tokens in the mask: the sort is stable) goes to
// rank[pair], and the histogram is written whole to blkcnt[blk][0 .. E), so nothing needs clearing
// beforehand.  lds: 3 * E ints (histogram, mask low and high words).
constexpr int kRouteThreads = 1024;
constexpr int kTokPerWave = kRouteTokens / (kRouteThreads / 64);  // 4
static_assert(kTokPerWave == 4 && kRouteTokens == 64, "one token per row of 16 lanes; 64-bit token masks");
constexpr int kRouteLdsInts = 3 * 1024;
template <int NPL>
MX_DEV void route_block(const float* __restrict__ logits, int64_t T, int E, int k, int renormalize,
                        int32_t* __restrict__ ids, float* __restrict__ wts, int32_t* __restrict__ blkcnt,
                        int32_t* __restrict__ rank, int64_t blk, int32_t* lds) {
  int32_t* hist = lds;
  uint32_t* mlo = reinterpret_cast<uint32_t*>(lds + E);
  uint32_t* mhi = reinterpret_cast<uint32_t*>(lds + 2 * E);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += kRouteThreads) {
    hist[e] = 0;
    mlo[e] = 0;
    mhi[e] = 0;
  }
  __syncthreads();
  const int64_t t0 = blk * kRouteTokens + wave * kTokPerWave;
  // this lane's pairs: token (local index within the block) and expert, -1 where the lane holds none
  constexpr bool ROWS = NPL <= 4;
  int pl[kTokPerWave], pe[kTokPerWave], pj[kTokPerWave];
#pragma unroll
  for (int i = 0; i < kTokPerWave; i++) pl[i] = -1;
  auto count = [&](int tl, int e) __attribute__((always_inline)) {
    atomicAdd(&hist[e], 1);
    if (tl < 32) atomicOr(&mlo[e], 1u << tl);
    else atomicOr(&mhi[e], 1u << (tl - 32));
  };
  bool rows = false;
  if constexpr (ROWS) {
    if (k <= 16) {
      rows = true;
      constexpr int NPR = 4 * NPL;  // E <= 16 * NPR
      const int q = lane & 15;
      const int64_t t = t0 + (lane >> 4);
      float val[NPR];
#pragma unroll
      for (int j = 0; j < NPR; j++) {
        const int idx = q + 16 * j;
        val[j] = t < T && idx < E ? logits[t * E + idx] : 0.f;
      }
      int my_id;
      float my_w;
      route_rows<NPR>(val, E, k, renormalize, my_id, my_w);
      if (t < T && q < k) {
        ids[t * k + q] = my_id;
        wts[t * k + q] = my_w;
        pl[0] = (int)(t - blk * kRouteTokens);
        pe[0] = my_id;
        pj[0] = q;
        count(pl[0], my_id);
      }
    }
  }
  if (!rows) {
    constexpr int NT = NPL <= 8 ? kTokPerWave : 2;  // tokens routed together
#pragma unroll
    for (int i0 = 0; i0 < kTokPerWave; i0 += NT) {
      if (t0 + i0 >= T) break;  // uniform per wave
      float val[NT][NPL];
#pragma unroll
      for (int i = 0; i < NT; i++) {
        const int64_t t = t0 + i0 + i;
#pragma unroll
        for (int j = 0; j < NPL; j++) {
          const int idx = lane + 64 * j;
          val[i][j] = t < T && idx < E ? logits[t * E + idx] : 0.f;
        }
      }
      int my_id[NT];
      float my_w[NT];
      route_tokens<NPL, NT>(val, E, k, renormalize, my_id, my_w);
#pragma unroll
      for (int i = 0; i < NT; i++) {
        const int64_t t = t0 + i0 + i;
        if (t < T && lane < k) {
          ids[t * k + lane] = my_id[i];
          wts[t * k + lane] = my_w[i];
          pl[i0 + i] = (int)(t - blk * kRouteTokens);
          pe[i0 + i] = my_id[i];
          pj[i0 + i] = lane;
          count(pl[i0 + i], my_id[i]);
        }
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kTokPerWave; i++)
    if (pl[i] >= 0) {
      const uint64_t m = ((uint64_t)mhi[pe[i]] << 32) | mlo[pe[i]];
      rank[(blk * kRouteTokens + pl[i]) * k + pj[i]] = __popcll(m & ((1ull << pl[i]) - 1ull));
    }
  for (int e = tid; e < E; e += kRouteThreads) blkcnt[blk * E + e] = hist[e];
}

template <int NPL>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(const float* __restrict__ logits, int64_t T, int E, int k,
                                                              int renormalize, int32_t* __restrict__ ids,
                                                              float* __restrict__ wts, int32_t* __restrict__ blkcnt,
                                                              int32_t* __restrict__ rank) {
  __shared__ int32_t lds[kRouteLdsInts];
  route_block<NPL>(logits, T, E, k, renormalize, ids, wts, blkcnt, rank, blockIdx.x, lds);
}

// The forward pass's front in one launch.  When the routing and the split workgroups all fit on the
// CUs at once (merged = 0), workgroups 0 .. nroute - 1 route one token block each and the others split
// the activations (16 waves each, with their own LDS staging; the routing histogram reuses the same
// LDS).  Otherwise (merged = 1) the grid has one workgroup per CU: the first min(nroute, grid) route
// the blocks dealt to them and then split groups 0 .. gsplit - 1, the others split the rest from the
// start, so that both kinds finish together.
template <int AF, int NPL>
__global__ __launch_bounds__(kRouteThreads) void front_kernel(const uint16_t* __restrict__ x, int64_t ldx, int64_t H,
                                                              int64_t nblk, uint8_t* __restrict__ xq, int64_t n,
                                                              const float* __restrict__ logits, int64_t T, int E, int k,
                                                              int renormalize, int32_t* __restrict__ ids,
                                                              float* __restrict__ wts, int32_t* __restrict__ blkcnt,
                                                              int32_t* __restrict__ rank, int nroute, int merged,
                                                              int64_t gsplit) {
  constexpr int REC = act_rec(AF), NW = kRouteThreads / 64;
  constexpr int kStage = 4096 > 32 * REC ? 4096 : 32 * REC;  // a wave's staging bytes
  static_assert(NW * kStage >= kRouteLdsInts * 4, "the routing tables fit the staging LDS");
  __shared__ __attribute__((aligned(16))) uint8_t smem[NW * kStage];
  const int wave = threadIdx.x >> 6;
  const int64_t ngroups = (n + 63) / 64;
  if (merged) {
    const int nr = nroute < (int)gridDim.x ? nroute : (int)gridDim.x;  // workgroups that route
    for (int b = blockIdx.x; b < nroute; b += gridDim.x) {
      route_block<NPL>(logits, T, E, k, renormalize, ids, wts, blkcnt, rank, b, reinterpret_cast<int32_t*>(smem));
      __syncthreads();  // the routing tables' last reads before the LDS holds split stages
    }
    if ((int)blockIdx.x < nr)
      xprep_waves<AF>(x, ldx, H, nblk, xq, n, (int64_t)blockIdx.x * NW + wave, gsplit, (int64_t)nr * NW,
                      smem + wave * kStage);
    else
      xprep_waves<AF>(x, ldx, H, nblk, xq, n, gsplit + (int64_t)(blockIdx.x - nr) * NW + wave, ngroups,
                      (int64_t)(gridDim.x - nr) * NW, smem + wave * kStage);
    return;
  }
  if ((int)blockIdx.x < nroute) {
    route_block<NPL>(logits, T, E, k, renormalize, ids, wts, blkcnt, rank, blockIdx.x, reinterpret_cast<int32_t*>(smem));
    return;
  }
  xprep_waves<AF>(x, ldx, H, nblk, xq, n, (int64_t)(blockIdx.x - nroute) * NW + wave, ngroups,
                  (int64_t)(gridDim.x - nroute) * NW, smem + wave * kStage);
}

// Pair placement, one workgroup of 1024 threads per block of kRouteTokens tokens.  blkcnt[b][e] holds
// the pairs of expert e among the tokens of block b (the routing histogram, read only here) and
// rank[pair] the pair's rank among the pairs of its expert within its block (token order).
//  (1) Every workgroup sums, per expert, the counts of the blocks before its own and of all blocks
//      (threads split the blocks, partial sums meet in LDS), then scans over experts: the exclusive
//      prefixes of the counts, of the counts padded to 32 and of the M tiles of BM and of BM2 rows.
//  (2) Workgroup 0 writes offsets, padded offsets and the tile counts; the workgroups share the
//      experts (expert e goes to workgroup e % gridDim.x; with few token blocks the grid has extra
//      workgroups, which hold no pairs) to write two tile lists (expert, first padded row,
//      valid rows) for M tiles of BM rows (first GEMM) and of BM2 rows (second GEMM; the list is
//      skipped when tiles2 is NULL) and the padding rows of each expert; workgroup 0 also writes 128
//      slack rows after the last expert (pair -1, token 0, weight 0), so a GEMM tile may read up to
//      128 rows past its expert's start.
//  (3) Each thread takes pairs of the block: rank = (pairs of that expert in earlier blocks) +
//      rank[pair]; it writes the compact order (sorted_pairs, may be NULL), the padded row (pair,
//      token, routing weight) and the pair's padded row (pair_prow, may be NULL; it may also be the
//      rank array itself, each entry read before its thread overwrites it).  Padding rows and pair rows
//      are disjoint, so the workgroups never write the same row.
__global__ __launch_bounds__(1024) void place_kernel(const int32_t* __restrict__ ids, const float* __restrict__ wts,
                                                     const int32_t* __restrict__ blkcnt, int64_t T, int nb, int k,
                                                     int E, int BM, int BM2, int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ poffsets, TileDesc* __restrict__ tiles,
                                                     int32_t* __restrict__ ntiles, TileDesc* __restrict__ tiles2,
                                                     int32_t* __restrict__ ntiles2, int32_t* __restrict__ sorted_pairs,
                                                     int32_t* __restrict__ prow_pair, int32_t* __restrict__ prow_tok,
                                                     float* __restrict__ prow_w, int32_t* pair_prow,
                                                     const int32_t* rank) {
  __shared__ int part_pre[1024], part_tot[1024];
  __shared__ int e_pre[1024], e_off[1024], e_poff[1024], e_tot[1024], e_toff[1024], e_toff2[1024];
  __shared__ int wsum[4][16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int blk = blockIdx.x;
  int es = 64;  // expert stride: power of two >= E, at least one wave
  while (es < E) es <<= 1;
  const int G = 1024 / es;  // block groups
  const int e = tid % es, grp = tid / es;
  const int per = (nb + G - 1) / G;
  const int b0 = min(nb, grp * per), b1 = min(nb, b0 + per);
  // this thread's pairs of the block (top_k <= 32: at most two per thread), loaded before phase (1)
  const int64_t pb0 = (int64_t)blk * kRouteTokens * k, npb = min((int64_t)kRouteTokens * k, T * k - pb0);
  int p_ex[2], p_rk[2];
  float p_wt[2];
#pragma unroll
  for (int u = 0; u < 2; u++) {
    const int64_t p = tid + 1024 * u;
    p_ex[u] = -1;
    if (p < npb) {
      p_ex[u] = ids[pb0 + p];
      p_wt[u] = wts[pb0 + p];
      p_rk[u] = rank[pb0 + p];
    }
  }
  // (1) partial sums over this thread's blocks, 16 independent loads at a time
  constexpr int kBatch = 16;
  int s_pre = 0, s_tot = 0;
  if (e < E)
    for (int bb = b0; bb < b1; bb += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; i++) v[i] = bb + i < b1 ? blkcnt[(int64_t)(bb + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kBatch; i++) {
        s_tot += v[i];
        s_pre += bb + i < blk ? v[i] : 0;
      }
    }
  part_pre[tid] = s_pre;
  part_tot[tid] = s_tot;
  __syncthreads();
  int v0 = 0, v1 = 0, v2 = 0, v3 = 0, pre = 0;
  if (grp == 0 && e < E) {
    int total = 0;
    for (int q = 0; q < G; q++) {
      pre += part_pre[q * es + e];
      total += part_tot[q * es + e];
    }
    v0 = total;
    v1 = (total + 31) & ~31;
    v2 = (total + BM - 1) / BM;
    v3 = (total + BM2 - 1) / BM2;
  }
  // scans over experts: thread e of group 0 (tid == e) holds expert e, every other thread zeros
  int x0 = v0, x1 = v1, x2 = v2, x3 = v3;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y0 = __shfl_up(x0, off), y1 = __shfl_up(x1, off), y2 = __shfl_up(x2, off), y3 = __shfl_up(x3, off);
    if (lane >= off) { x0 += y0; x1 += y1; x2 += y2; x3 += y3; }
  }
  if (lane == 63) { wsum[0][wave] = x0; wsum[1][wave] = x1; wsum[2][wave] = x2; wsum[3][wave] = x3; }
  __syncthreads();
  int p0 = 0, p1 = 0, p2 = 0, p3 = 0;
  for (int q = 0; q < wave; q++) { p0 += wsum[0][q]; p1 += wsum[1][q]; p2 += wsum[2][q]; p3 += wsum[3][q]; }
  x0 += p0; x1 += p1; x2 += p2; x3 += p3;  // inclusive scans over threads 0..tid
  if (grp == 0 && e < E) {
    e_pre[e] = pre;
    e_off[e] = x0 - v0;
    e_poff[e] = x1 - v1;
    e_tot[e] = v0;
    e_toff[e] = x2 - v2;
    e_toff2[e] = x3 - v3;
  }
  // (2) offsets and counts by workgroup 0's expert threads; tiles and padding rows of expert ee by
  // workgroup ee % nb, its waves taking those experts in turn with one lane per tile or row
  if (blk == 0 && grp == 0 && e < E) {
    offsets[e] = x0 - v0;
    poffsets[e] = x1 - v1;
    if (e == E - 1) {
      offsets[E] = x0;
      poffsets[E] = x1;
      *ntiles = x2;
      if (tiles2) *ntiles2 = x3;
    }
  }
  __syncthreads();
  const int nwg = gridDim.x;  // at least nb (workgroups past nb have no pairs and only write tables)
  for (int ee = blk + wave * nwg; ee < E; ee += 16 * nwg) {
    const int poff = e_poff[ee], total = e_tot[ee], toff = e_toff[ee];
    const int ntl = (total + BM - 1) / BM, pad = ((total + 31) & ~31) - total;
    for (int i = lane; i < ntl; i += 64) tiles[toff + i] = TileDesc{ee, poff + i * BM, min(BM, total - i * BM), 0};
    if (tiles2) {
      const int toff2 = e_toff2[ee], ntl2 = (total + BM2 - 1) / BM2;
      for (int i = lane; i < ntl2; i += 64) tiles2[toff2 + i] = TileDesc{ee, poff + i * BM2, min(BM2, total - i * BM2), 0};
    }
    if (lane < pad) {
      const int r = poff + total + lane;
      prow_pair[r] = -1;
      prow_tok[r] = 0;
      prow_w[r] = 0.f;
    }
  }
  if (blk == 0 && tid < 128) {  // slack rows after the last expert
    const int r = e_poff[E - 1] + ((e_tot[E - 1] + 31) & ~31) + tid;
    prow_pair[r] = -1;
    prow_tok[r] = 0;
    prow_w[r] = 0.f;
  }
  // (3) the block's pairs, from the ranks the routing wrote
#pragma unroll
  for (int u = 0; u < 2; u++) {
    const int ex = p_ex[u];
    if (ex < 0) continue;
    const int64_t pair = pb0 + tid + 1024 * u;
    const int rk = e_pre[ex] + p_rk[u];
    if (sorted_pairs) sorted_pairs[e_off[ex] + rk] = (int32_t)pair;
    const int r = e_poff[ex] + rk;
    prow_pair[r] = (int32_t)pair;
    prow_tok[r] = (int32_t)(pair / k);
    prow_w[r] = p_wt[u];
    if (pair_prow) pair_prow[pair] = r;
  }
}

// E <= 64 * NPL: the NPL of a routing instantiation, or 0 past 1024 experts
inline int route_npl(int E) { return E <= 64 ? 1 : E <= 128 ? 2 : E <= 256 ? 4 : E <= 512 ? 8 : E <= 1024 ? 16 : 0; }

template <int AF>
void launch_front_af(const void* x, int64_t T, int64_t ldx, const MoeGeom& g, void* xq, const float* logits, int E,
                     int k, int renormalize, int32_t* ids, float* w, int32_t* blkcnt, int32_t* rank,
                     hipStream_t stream) {
  const int64_t nblk = 2 * g.nkt1;
  const int64_t n = T * nblk;
  const int nroute = (int)cdiv(T, kRouteTokens);
  // Split workgroups: one wave per group of 64 blocks when they fit beside the routing workgroups on
  // the CUs at once (one 1024-thread workgroup per CU).  Otherwise one workgroup per CU; a routing
  // workgroup's waves then take fewer groups, the routing of a block costing about NPL / 2 groups.
  constexpr int kCus = 256, NW = kRouteThreads / 64;
  const int64_t ngroups = cdiv(n, 64);
  const int64_t nx = cdiv(ngroups, NW);
  const int merged = nroute + nx > kCus ? 1 : 0;
  int64_t gsplit = ngroups;
  if (merged && nroute < kCus) {
    const int64_t avg = ngroups / (kCus * NW);           // groups per wave, all waves alike
    const int64_t per = avg - route_npl(E) / 2;          // per routing wave
    gsplit = per > 0 ? (int64_t)nroute * NW * per : 0;
  }
  const dim3 grid((unsigned)(merged ? kCus : nroute + nx)), block(kRouteThreads);
#define MX_FRONT(NPL)                                                                                                   \
  hipLaunchKernelGGL((front_kernel<AF, NPL>), grid, block, 0, stream, (const uint16_t*)x, ldx, g.H, nblk, (uint8_t*)xq, n, \
                     logits, T, E, k, renormalize, ids, w, blkcnt, rank, nroute, merged, gsplit)
  switch (route_npl(E)) {
    case 1: MX_FRONT(1); break;
    case 2: MX_FRONT(2); break;
    case 4: MX_FRONT(4); break;
    case 8: MX_FRONT(8); break;
    default: MX_FRONT(16); break;
  }
#undef MX_FRONT
}

}  // namespace

int launch_front(int af, const void* x, int64_t T, int64_t ldx, const MoeGeom& g, void* xq, const float* logits, int E,
                 int k, int renormalize, int32_t* ids, float* w, int32_t* blkcnt, int32_t* rank, hipStream_t stream) {
  if (T > 0) {
    if (af == kActMxfp8)
      launch_front_af<kActMxfp8>(x, T, ldx, g, xq, logits, E, k, renormalize, ids, w, blkcnt, rank, stream);
    else if (af == kActMxfp4)
      launch_front_af<kActMxfp4>(x, T, ldx, g, xq, logits, E, k, renormalize, ids, w, blkcnt, rank, stream);
    else
      launch_front_af<kActBf16>(x, T, ldx, g, xq, logits, E, k, renormalize, ids, w, blkcnt, rank, stream);
  }
  return hipGetLastError() == hipSuccess ? MXFP4_OK : MXFP4_ERR_DEVICE;
}

int launch_route(const float* logits, int64_t T, int E, int k, int renormalize, int32_t* ids, float* w,
                 int32_t* blkcnt, int32_t* rank, hipStream_t stream) {
  const dim3 grid((unsigned)cdiv(T, kRouteTokens)), block(kRouteThreads);
#define MX_ROUTE(NPL) \
  hipLaunchKernelGGL(route_kernel<NPL>, grid, block, 0, stream, logits, T, E, k, renormalize, ids, w, blkcnt, rank)
  if (T > 0) {
    switch (route_npl(E)) {
      case 1: MX_ROUTE(1); break;
      case 2: MX_ROUTE(2); break;
      case 4: MX_ROUTE(4); break;
      case 8: MX_ROUTE(8); break;
      default: MX_ROUTE(16); break;
    }
  }
#undef MX_ROUTE
  return hipGetLastError() == hipSuccess ? MXFP4_OK : MXFP4_ERR_DEVICE;
}

int launch_place(const int32_t* ids, const float* w, int32_t* blkcnt, const int32_t* rank, int64_t T, int k, int E,
                 int BM, int BM2, int32_t* offsets, int32_t* poffsets, int32_t* sorted_pairs, int32_t* prow_pair,
                 int32_t* prow_tok, float* prow_w, int32_t* pair_prow, void* tiles, int32_t* ntiles, void* tiles2,
                 int32_t* ntiles2, hipStream_t stream) {
  const int nb = (int)cdiv(T, kRouteTokens);
  // one workgroup per token block, and at least one (the tables are written even without tokens); with
  // few blocks, more workgroups (up to one expert per wave) share the tile lists and padding rows
  int nwg = nb > 0 ? nb : 1;
  const int by_experts = (int)cdiv(E, 16) < 16 ? (int)cdiv(E, 16) : 16;
  if (nwg < by_experts) nwg = by_experts;
  hipLaunchKernelGGL(place_kernel, dim3((unsigned)nwg), dim3(1024), 0, stream, ids, w, blkcnt, T, nb, k, E,
                     BM, BM2, offsets, poffsets, (TileDesc*)tiles, ntiles, (TileDesc*)tiles2, ntiles2, sorted_pairs, prow_pair,
                     prow_tok, prow_w, pair_prow, rank);
  return hipGetLastError() == hipSuccess ? MXFP4_OK : MXFP4_ERR_DEVICE;
}
