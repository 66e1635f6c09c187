// C ABI of the library: argument validation (before any device work), workspace carving and the
// stream-ordered launch sequence.  Declarations and the contract of every entry point are in
// include/mxfp4moe.h.
#include <hip/hip_runtime_api.h>

#include <cstring>

#include "internal.h"

#define MX_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kMaxE = 1024;
constexpr int64_t kMaxDim = int64_t(1) << 40;  // bound on any matrix dimension (keeps sizes in 64 bits)
constexpr int kMaxTopK = 32;

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
inline hipStream_t S(void* s) { return (hipStream_t)s; }

int check_dims(const mxfp4_moe_dims* d) {
  if (!d) return MXFP4_ERR_NULL;
  if (d->E < 1 || d->H < 32 || d->I < 32 || d->H % 32 || d->I % 32) return MXFP4_ERR_SHAPE;
  if (d->has_bias != 0 && d->has_bias != 1) return MXFP4_ERR_SHAPE;
  if ((int64_t)d->E * 2 * d->I > (1LL << 31) || (int64_t)d->E * d->H > (1LL << 31)) return MXFP4_ERR_SHAPE;
  return MXFP4_OK;
}

bool valid_layout(uint32_t layout) {
  return layout == MXFP4_LAYOUT_GFX950 || layout == MXFP4_LAYOUT_STD_W31 || layout == MXFP4_LAYOUT_SCALE_TILED ||
         layout == (MXFP4_LAYOUT_STD_W31 | MXFP4_LAYOUT_SCALE_TILED);
}

void standard_sizes(const mxfp4_moe_dims* d, uint32_t layout, size_t sz[6]) {
  const int64_t E = d->E, H = d->H, I = d->I;
  const bool tiled = layout & MXFP4_LAYOUT_SCALE_TILED;
  // the order of the pages' conversion result: w13, w2, w13 scales, w2 scales, b13, b2
  sz[0] = (size_t)(E * 2 * I * (H / 2));
  sz[1] = (size_t)(E * H * (I / 2));
  if (tiled) {
    sz[2] = (size_t)(E * cdiv(2 * I, 128) * cdiv(H / 32, 4) * 512);
    sz[3] = (size_t)(E * cdiv(H, 128) * cdiv(I / 32, 4) * 512);
  } else {
    sz[2] = (size_t)(E * 2 * I * (H / 32));
    sz[3] = (size_t)(E * H * (I / 32));
  }
  sz[4] = d->has_bias ? (size_t)(E * 2 * I * 2) : 0;
  sz[5] = d->has_bias ? (size_t)(E * H * 2) : 0;
}

size_t standard_offsets(const mxfp4_moe_dims* d, uint32_t layout, size_t off[6]) {
  size_t sz[6];
  standard_sizes(d, layout, sz);
  size_t p = 0;
  for (int i = 0; i < 6; i++) {
    off[i] = p;
    p = (size_t)align256((int64_t)(p + sz[i]));
  }
  return p;
}

// Row groups of 32 per M tile of the first GEMM, from the mean rows per expert.
int choose_nrg1(int64_t P, int64_t E) {
  const int64_t avg = P / (E > 0 ? E : 1);
  if (avg < 48) return 1;
  if (avg < 160) return 2;
  return 4;
}

// The same for the second GEMM.  With one-term operands (the quantized-activation formats) its 64-row
// tiles measured fastest once experts average 48 rows.  With the bf16 path's three-term operand a
// 64-row tile needs more registers than two workgroups per CU leave, and 32-row tiles at two workgroups
// per CU measured fastest up to a few hundred rows per expert; from an average of 160 rows the first
// GEMM's 128-row shape (one workgroup per CU) is a little faster.
int choose_nrg2(int64_t P, int64_t E, int32_t act) {
  const int64_t avg = P / (E > 0 ? E : 1);
  if (act == MXFP4_ACT_BF16) return avg < 160 ? 1 : 4;
  return avg < 48 ? 1 : 2;
}

struct RouteWs {
  uint64_t blkcnt, rank, poffsets, prow_pair, prow_tok, prow_w, tiles, ntiles, total;
  int64_t max_tiles;
};

RouteWs route_ws(int64_t T, int64_t E, int64_t k) {
  RouteWs w;
  const int64_t P = T * k;
  const int64_t nrows = ((P + 31 * E + 31) / 32) * 32 + 128;
  w.max_tiles = cdiv(P, 32) + E;
  uint64_t p = 0;
  auto take = [&](uint64_t bytes) { uint64_t o = p; p = align256((int64_t)(p + bytes)); return o; };
  w.blkcnt = take(4 * cdiv(T, kRouteTokens) * E + 4);
  w.rank = take(4 * P + 4);
  w.poffsets = take(4 * (E + 1));
  w.prow_pair = take(4 * nrows);
  w.prow_tok = take(4 * nrows);
  w.prow_w = take(4 * nrows);
  w.tiles = take(16 * w.max_tiles);
  w.ntiles = take(16);
  w.total = p;
  return w;
}

int check_route_args(int64_t T, int32_t E, int32_t top_k) {
  if (T < 0 || E < 1 || E > kMaxE || top_k < 1 || top_k > E || top_k > kMaxTopK) return MXFP4_ERR_SHAPE;
  if (T > (1LL << 31) || T * top_k + 32LL * E + 256 > (1LL << 31) - 1) return MXFP4_ERR_SHAPE;
  return MXFP4_OK;
}

}  // namespace

MX_API const char* mxfp4_status_str(int status) {
  switch (status) {
    case MXFP4_OK: return "ok";
    case MXFP4_ERR_NULL: return "a required pointer is NULL";
    case MXFP4_ERR_SHAPE: return "a size or dimension is out of range";
    case MXFP4_ERR_ALIGN: return "a pointer or stride is misaligned";
    case MXFP4_ERR_WORKSPACE: return "workspace or output buffer too small";
    case MXFP4_ERR_LAYOUT: return "unknown layout, or packed weights that do not match the dimensions";
    case MXFP4_ERR_DEVICE: return "a HIP call or kernel launch failed";
    default: return "unknown status";
  }
}

MX_API uint32_t mxfp4_version(void) { return (1u << 16) | 0u; }

MX_API size_t mxfp4_tiled_scale_bytes(int64_t M, int64_t K) {
  if (M < 0 || K < 32 || K % 32 || M > kMaxDim || K > kMaxDim) return 0;
  return (size_t)(cdiv(M, 128) * cdiv(K / 32, 4) * 512);
}

MX_API int mxfp4_quantize(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, void* q_u8, void* scale_flat_u8,
                          void* scale_tiled_u8, void* stream) {
  if (M < 0 || K < 32 || K % 32 || ldx < K || ldx % 8 || ldx > kMaxDim) return MXFP4_ERR_SHAPE;
  if (M > kMaxDim / ldx) return MXFP4_ERR_SHAPE;
  if (M == 0) return MXFP4_OK;
  if (!x_bf16 || !q_u8) return MXFP4_ERR_NULL;
  if (!aligned(x_bf16, 16) || !aligned(q_u8, 4) || (scale_tiled_u8 && !aligned(scale_tiled_u8, 16)))
    return MXFP4_ERR_ALIGN;
  return launch_quantize(x_bf16, M, K, ldx, q_u8, scale_flat_u8, scale_tiled_u8, S(stream));
}

MX_API size_t nvfp4_tiled_scale_bytes(int64_t M, int64_t K) {
  if (M < 0 || K < 16 || K % 16 || M > kMaxDim || K > kMaxDim) return 0;
  return (size_t)(cdiv(M, 128) * cdiv(K / 16, 4) * 512);
}

MX_API int nvfp4_quantize(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, float global_scale, void* q_u8,
                          void* scale_flat_u8, void* scale_tiled_u8, void* stream) {
  if (M < 0 || K < 16 || K % 16 || ldx < K || ldx % 8 || ldx > kMaxDim) return MXFP4_ERR_SHAPE;
  if (M > kMaxDim / ldx) return MXFP4_ERR_SHAPE;
  // a positive, finite binary32 global scale (the comparison also rejects NaN)
  if (!(global_scale > 0.0f && global_scale <= 3.40282347e38f)) return MXFP4_ERR_SHAPE;
  if (M == 0) return MXFP4_OK;
  if (!x_bf16 || !q_u8) return MXFP4_ERR_NULL;
  if (!aligned(x_bf16, 16) || !aligned(q_u8, 4) || (scale_tiled_u8 && !aligned(scale_tiled_u8, 16)))
    return MXFP4_ERR_ALIGN;
  return launch_nvfp4_quantize(x_bf16, M, K, ldx, global_scale, q_u8, scale_flat_u8, scale_tiled_u8, S(stream));
}

MX_API size_t mxfp4_repack_bytes(const mxfp4_moe_dims* d, uint32_t layout) {
  if (check_dims(d) != MXFP4_OK || !valid_layout(layout)) return 0;
  if (layout == MXFP4_LAYOUT_GFX950) return (size_t)blob_offsets(moe_geom(d->E, d->H, d->I), d->has_bias).total;
  size_t off[6];
  return standard_offsets(d, layout, off);
}

MX_API int mxfp4_repack_offsets(const mxfp4_moe_dims* d, uint32_t layout, size_t offsets_out[6]) {
  int st = check_dims(d);
  if (st) return st;
  if (!offsets_out) return MXFP4_ERR_NULL;
  if (!valid_layout(layout) || layout == MXFP4_LAYOUT_GFX950) return MXFP4_ERR_LAYOUT;
  standard_offsets(d, layout, offsets_out);
  return MXFP4_OK;
}

MX_API int mxfp4_repack_weights(const mxfp4_moe_dims* d, const void* w13_q, const void* w13_s, const void* w2_q,
                                const void* w2_s, const void* b13, const void* b2, int32_t bias_is_fp32,
                                uint32_t layout, void* out, size_t out_bytes, void* stream) {
  int st = check_dims(d);
  if (st) return st;
  if (!valid_layout(layout)) return MXFP4_ERR_LAYOUT;
  if (!w13_q || !w13_s || !w2_q || !w2_s || !out) return MXFP4_ERR_NULL;
  if (d->has_bias && (!b13 || !b2)) return MXFP4_ERR_NULL;
  if (!aligned(w13_q, 16) || !aligned(w2_q, 16) || !aligned(out, 256)) return MXFP4_ERR_ALIGN;
  if (d->has_bias && (!aligned(b13, bias_is_fp32 ? 4 : 2) || !aligned(b2, bias_is_fp32 ? 4 : 2)))
    return MXFP4_ERR_ALIGN;
  const size_t need = mxfp4_repack_bytes(d, layout);
  if (out_bytes < need) return MXFP4_ERR_WORKSPACE;
  const MoeGeom g = moe_geom(d->E, d->H, d->I);
  if (layout == MXFP4_LAYOUT_GFX950)
    return launch_repack_gfx950(g, blob_offsets(g, d->has_bias), d->has_bias, w13_q, w13_s, w2_q, w2_s, b13, b2,
                                bias_is_fp32, out, S(stream));
  size_t off[6];
  standard_offsets(d, layout, off);
  return launch_repack_standard(g, d->has_bias, w13_q, w13_s, w2_q, w2_s, b13, b2, bias_is_fp32,
                                (layout & MXFP4_LAYOUT_STD_W31) != 0, (layout & MXFP4_LAYOUT_SCALE_TILED) != 0, off, out,
                                S(stream));
}

static int read_header(const void* packed, BlobHeader* h, hipStream_t stream) {
  if (hipMemcpyAsync(h, packed, sizeof(BlobHeader), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return MXFP4_ERR_DEVICE;
  if (hipStreamSynchronize(stream) != hipSuccess) return MXFP4_ERR_DEVICE;
  return MXFP4_OK;
}

static int header_matches(const mxfp4_moe_dims* d, const BlobHeader& h) {
  if (std::memcmp(h.magic, MX_BLOB_MAGIC, 8) != 0 || h.version != MX_BLOB_VERSION) return 0;
  if (h.E != d->E || h.H != d->H || h.I != d->I || h.has_bias != d->has_bias) return 0;
  const BlobOffsets o = blob_offsets(moe_geom(d->E, d->H, d->I), d->has_bias);
  return h.off_w13q == o.w13q && h.off_w13s == o.w13s && h.off_w2q == o.w2q && h.off_w2s == o.w2s &&
         h.off_b13 == o.b13 && h.off_b2 == o.b2 && h.total == o.total;
}

MX_API int mxfp4_check_packed(const mxfp4_moe_dims* d, const void* packed, void* stream) {
  int st = check_dims(d);
  if (st) return st;
  if (!packed) return MXFP4_ERR_NULL;
  if (!aligned(packed, 256)) return MXFP4_ERR_ALIGN;
  BlobHeader h;
  st = read_header(packed, &h, S(stream));
  if (st) return st;
  return header_matches(d, h) ? MXFP4_OK : MXFP4_ERR_LAYOUT;
}

MX_API int mxfp4_unpack_weights(const mxfp4_moe_dims* d, const void* packed, void* w13_q, void* w13_s, void* w2_q,
                                void* w2_s, void* b13_bf16, void* b2_bf16, void* stream) {
  int st = check_dims(d);
  if (st) return st;
  if (!packed || !w13_q || !w13_s || !w2_q || !w2_s) return MXFP4_ERR_NULL;
  if (!aligned(packed, 256) || !aligned(w13_q, 16) || !aligned(w2_q, 16)) return MXFP4_ERR_ALIGN;
  if ((b13_bf16 && !aligned(b13_bf16, 2)) || (b2_bf16 && !aligned(b2_bf16, 2))) return MXFP4_ERR_ALIGN;
  BlobHeader h;
  st = read_header(packed, &h, S(stream));
  if (st) return st;
  if (!header_matches(d, h)) return MXFP4_ERR_LAYOUT;
  const MoeGeom g = moe_geom(d->E, d->H, d->I);
  return launch_unpack_gfx950(g, blob_offsets(g, d->has_bias), d->has_bias, packed, w13_q, w13_s, w2_q, w2_s, b13_bf16,
                              b2_bf16, S(stream));
}

// ------------------------------------------------------------------------------------------------
// Dense linear layer.

static int check_linear_dims(int64_t N, int64_t K) {
  if (N < 32 || K < 32 || N % 32 || K % 32 || N > (1 << 20) || K > (1 << 20)) return MXFP4_ERR_SHAPE;
  return MXFP4_OK;
}

MX_API size_t mxfp4_linear_pack_bytes(int64_t N, int64_t K, int32_t has_bias) {
  if (check_linear_dims(N, K) != MXFP4_OK || (has_bias != 0 && has_bias != 1)) return 0;
  return (size_t)linear_offsets(moe_geom(1, N, K), has_bias != 0).total;
}

MX_API int mxfp4_linear_pack(int64_t N, int64_t K, const void* w_q, const void* w_s, const void* bias,
                             int32_t bias_is_fp32, void* out, size_t out_bytes, void* stream) {
  int st = check_linear_dims(N, K);
  if (st) return st;
  if (!w_q || !w_s || !out) return MXFP4_ERR_NULL;
  if (!aligned(w_q, 16) || !aligned(out, 256) || (bias && !aligned(bias, bias_is_fp32 ? 4 : 2))) return MXFP4_ERR_ALIGN;
  const MoeGeom g = moe_geom(1, N, K);
  const LinearOffsets o = linear_offsets(g, bias != nullptr);
  if (out_bytes < o.total) return MXFP4_ERR_WORKSPACE;
  return launch_pack_linear(g, o, bias != nullptr, w_q, w_s, bias, bias_is_fp32, out, S(stream));
}

MX_API size_t mxfp4_linear_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (check_linear_dims(N, K) != MXFP4_OK || M < 0 || M > (1LL << 31)) return 0;
  return (size_t)linear_ws(M, moe_geom(1, N, K)).total;
}

MX_API int mxfp4_linear_forward(const void* packed, int64_t N, int64_t K, int32_t has_bias, const void* x_bf16,
                                int64_t M, int64_t ldx, void* y_bf16, void* workspace, size_t workspace_bytes,
                                void* stream) {
  int st = check_linear_dims(N, K);
  if (st) return st;
  if (M < 0 || M > (1LL << 31) || ldx < K || ldx % 8 || (has_bias != 0 && has_bias != 1)) return MXFP4_ERR_SHAPE;
  const MoeGeom g = moe_geom(1, N, K);
  const LinearWs w = linear_ws(M, g);
  // the GEMM's copy sources are 32-bit byte offsets into the activation operand
  if ((uint64_t)w.nrg * g.nkt2 * 64 * kMaxSlot >= (1ULL << 32)) return MXFP4_ERR_SHAPE;
  if (M == 0) return MXFP4_OK;
  if (!packed || !x_bf16 || !y_bf16 || !workspace) return MXFP4_ERR_NULL;
  if (!aligned(packed, 256) || !aligned(x_bf16, 16) || !aligned(y_bf16, 16) || !aligned(workspace, 256))
    return MXFP4_ERR_ALIGN;
  if (workspace_bytes < w.total) return MXFP4_ERR_WORKSPACE;
  const LinearOffsets o = linear_offsets(g, has_bias != 0);
  const uint8_t* blob = (const uint8_t*)packed;
  uint8_t* ws = (uint8_t*)workspace;
  if ((st = launch_linear_prep(x_bf16, M, ldx, g, w, ws, S(stream)))) return st;
  GemmArgs a = {};
  a.wq = blob + o.wq;
  a.ws = blob + o.ws;
  a.bias = has_bias ? (const uint16_t*)(blob + o.bias) : nullptr;
  a.xq = ws + w.actq;
  a.xs = ws + w.acts;
  a.prow_w = (const float*)(ws + w.roww);
  a.tiles = (const TileDesc*)(ws + w.tiles);
  a.ntiles = (const int32_t*)(ws + w.ntiles);
  a.ydense = (uint16_t*)y_bf16;
  a.nkt = (int32_t)g.nkt2;
  a.ncb = (int32_t)g.ncb2;
  a.ntl = (int32_t)g.nht;
  a.nkt2 = (int32_t)g.nkt2;
  a.I = (int32_t)K;
  a.H = (int32_t)N;
  return launch_gemm2(MXFP4_ACT_BF16, 1, a, w.nrg, S(stream));
}

MX_API size_t moe_mxfp4_route_workspace_bytes(int64_t T, int32_t E, int32_t top_k) {
  if (check_route_args(T, E, top_k) != MXFP4_OK) return 0;
  return (size_t)route_ws(T, E, top_k).total;
}

MX_API int moe_mxfp4_route(const float* router_logits, int64_t T, int32_t E, int32_t top_k, int32_t renormalize,
                           int32_t* topk_ids, float* topk_w, int32_t* expert_offsets, int32_t* sorted_pairs,
                           void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_route_args(T, E, top_k);
  if (st) return st;
  if (!expert_offsets || !workspace) return MXFP4_ERR_NULL;
  if (T > 0 && (!router_logits || !topk_ids || !topk_w || !sorted_pairs)) return MXFP4_ERR_NULL;
  if (!aligned(router_logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4) || !aligned(expert_offsets, 4) ||
      !aligned(sorted_pairs, 4) || !aligned(workspace, 256))
    return MXFP4_ERR_ALIGN;
  const RouteWs w = route_ws(T, E, top_k);
  if (workspace_bytes < w.total) return MXFP4_ERR_WORKSPACE;
  uint8_t* ws = (uint8_t*)workspace;
  int32_t* blkcnt = (int32_t*)(ws + w.blkcnt);
  int32_t* rank = (int32_t*)(ws + w.rank);
  if ((st = launch_route(router_logits, T, E, top_k, renormalize, topk_ids, topk_w, blkcnt, rank, S(stream)))) return st;
  return launch_place(topk_ids, topk_w, blkcnt, rank, T, top_k, E, 32, 32, expert_offsets, (int32_t*)(ws + w.poffsets),
                      sorted_pairs, (int32_t*)(ws + w.prow_pair), (int32_t*)(ws + w.prow_tok), (float*)(ws + w.prow_w),
                      nullptr, ws + w.tiles, (int32_t*)(ws + w.ntiles), nullptr, nullptr, S(stream));
}

MX_API size_t moe_mxfp4_workspace_bytes(const mxfp4_moe_dims* d, int64_t T, int32_t top_k) {
  if (check_dims(d) != MXFP4_OK || check_route_args(T, d->E, top_k) != MXFP4_OK) return 0;
  return (size_t)fwd_ws(moe_geom(d->E, d->H, d->I), T, top_k).total;
}

int forward_impl(const mxfp4_moe_dims* d, int32_t act_format, const void* packed_gfx950, const void* x_bf16,
                 int64_t T, int64_t ldx, const float* router_logits, int32_t top_k, int32_t renormalize, void* y_bf16,
                 int32_t* topk_ids, float* topk_w, void* workspace, size_t workspace_bytes, hipStream_t s,
                 void* const* events, int32_t n_events) {
  int st = check_dims(d);
  if (st) return st;
  if (act_format != MXFP4_ACT_BF16 && act_format != MXFP4_ACT_MXFP8 && act_format != MXFP4_ACT_MXFP4)
    return MXFP4_ERR_LAYOUT;
  if ((st = check_route_args(T, d->E, top_k))) return st;
  if (ldx < d->H || ldx % 8) return MXFP4_ERR_SHAPE;
  if (n_events < 0 || (n_events > 0 && !events)) return MXFP4_ERR_NULL;
  if (T == 0) return MXFP4_OK;
  if (!packed_gfx950 || !x_bf16 || !router_logits || !y_bf16 || !workspace) return MXFP4_ERR_NULL;
  if (!aligned(packed_gfx950, 256) || !aligned(x_bf16, 16) || !aligned(router_logits, 4) || !aligned(y_bf16, 16) ||
      !aligned(workspace, 256) || (topk_ids && !aligned(topk_ids, 4)) || (topk_w && !aligned(topk_w, 4)))
    return MXFP4_ERR_ALIGN;
  const MoeGeom g = moe_geom(d->E, d->H, d->I);
  const FwdWs w = fwd_ws(g, T, top_k);
  // the GEMMs' copy sources are 32-bit byte offsets into the activation buffers
  if ((uint64_t)T * g.nkt1 * kMaxRec >= (1ULL << 32) ||
      (uint64_t)(w.nrows_alloc / 32) * g.nkt2 * 64 * kMaxSlot >= (1ULL << 32))
    return MXFP4_ERR_SHAPE;
  if (workspace_bytes < w.total) return MXFP4_ERR_WORKSPACE;
  const BlobOffsets o = blob_offsets(g, d->has_bias);
  uint8_t* ws = (uint8_t*)workspace;
  const int64_t P = T * top_k;
  int32_t* ids = topk_ids ? topk_ids : (int32_t*)(ws + w.ids);
  float* wts = topk_w ? topk_w : (float*)(ws + w.w);
  const int NRG1 = choose_nrg1(P, g.E), NRG2 = choose_nrg2(P, g.E, act_format);
  int ev = 0;
  auto mark = [&]() -> int {
    if (ev < n_events && hipEventRecord((hipEvent_t)events[ev], s) != hipSuccess) return MXFP4_ERR_DEVICE;
    ev++;
    return MXFP4_OK;
  };
  if ((st = mark())) return st;
  // the pairs' in-block ranks go to pair_prow, which the placement overwrites with their rows
  int32_t* pair_prow = (int32_t*)(ws + w.pair_prow);
  if ((st = launch_front(act_format, x_bf16, T, ldx, g, ws + w.xq, router_logits, (int)g.E, top_k, renormalize, ids,
                          wts, (int32_t*)(ws + w.blkcnt), pair_prow, s)) ||
      (st = mark()))
    return st;
  if ((st = launch_place(ids, wts, (int32_t*)(ws + w.blkcnt), pair_prow, T, top_k, (int)g.E, 32 * NRG1, 32 * NRG2,
                         (int32_t*)(ws + w.offsets), (int32_t*)(ws + w.poffsets), nullptr, (int32_t*)(ws + w.prow_pair),
                         (int32_t*)(ws + w.prow_tok), (float*)(ws + w.prow_w), pair_prow,
                         ws + w.tiles, (int32_t*)(ws + w.ntiles), ws + w.tiles2, (int32_t*)(ws + w.ntiles2), s)) ||
      (st = mark()))
    return st;
  const uint8_t* blob = (const uint8_t*)packed_gfx950;
  GemmArgs a1 = {blob + o.w13q, blob + o.w13s, d->has_bias ? (const uint16_t*)(blob + o.b13) : nullptr,
                 ws + w.xq, nullptr, (const int32_t*)(ws + w.prow_tok), (const int32_t*)(ws + w.prow_pair),
                 (const float*)(ws + w.prow_w), (const TileDesc*)(ws + w.tiles), (const int32_t*)(ws + w.ntiles),
                 ws + w.actq, ws + w.acts, nullptr, nullptr, nullptr, (int32_t)g.nkt1, (int32_t)g.ncb1, (int32_t)g.nit,
                 (int32_t)g.nkt2, (int32_t)g.nkt1, (int32_t)g.I, (int32_t)g.H};
  if ((st = launch_gemm1(act_format, NRG1, a1, w.max_tiles, s)) || (st = mark())) return st;
  GemmArgs a2 = a1;
  a2.wq = blob + o.w2q;
  a2.ws = blob + o.w2s;
  a2.bias = d->has_bias ? (const uint16_t*)(blob + o.b2) : nullptr;
  a2.xq = ws + w.actq;
  a2.xs = ws + w.acts;
  a2.o16 = (uint16_t*)(ws + w.o16);
  a2.osc = ws + w.osc;
  a2.nkt = (int32_t)g.nkt2;
  a2.ncb = (int32_t)g.ncb2;
  a2.ntl = (int32_t)g.nht;
  a2.tiles = (const TileDesc*)(ws + w.tiles2);
  a2.ntiles = (const int32_t*)(ws + w.ntiles2);
  if ((st = launch_gemm2(act_format, NRG2, a2, w.max_tiles, s)) || (st = mark())) return st;
  if ((st = launch_combine((const uint16_t*)(ws + w.o16), ws + w.osc, (const int32_t*)(ws + w.pair_prow), y_bf16, T, g.H,
                           top_k, s)) ||
      (st = mark()))
    return st;
  return MXFP4_OK;
}

MX_API int moe_mxfp4_forward(const mxfp4_moe_dims* d, const void* packed_gfx950, const void* x_bf16, int64_t T,
                             int64_t ldx, const float* router_logits, int32_t top_k, int32_t renormalize, void* y_bf16,
                             int32_t* topk_ids, float* topk_w, void* workspace, size_t workspace_bytes, void* stream) {
  return forward_impl(d, MXFP4_ACT_BF16, packed_gfx950, x_bf16, T, ldx, router_logits, top_k, renormalize, y_bf16,
                      topk_ids, topk_w, workspace, workspace_bytes, S(stream), nullptr, 0);
}

MX_API int moe_mxfp4_forward_act(const mxfp4_moe_dims* d, int32_t act_format, const void* packed_gfx950,
                                 const void* x_bf16, int64_t T, int64_t ldx, const float* router_logits, int32_t top_k,
                                 int32_t renormalize, void* y_bf16, int32_t* topk_ids, float* topk_w, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return forward_impl(d, act_format, packed_gfx950, x_bf16, T, ldx, router_logits, top_k, renormalize, y_bf16, topk_ids,
                      topk_w, workspace, workspace_bytes, S(stream), nullptr, 0);
}

MX_API int moe_mxfp4_forward_profiled(const mxfp4_moe_dims* d, int32_t act_format, const void* packed_gfx950,
                                      const void* x_bf16, int64_t T, int64_t ldx, const float* router_logits,
                                      int32_t top_k, int32_t renormalize, void* y_bf16, int32_t* topk_ids,
                                      float* topk_w, void* workspace, size_t workspace_bytes, void* stream,
                                      void* const* events, int32_t n_events) {
  return forward_impl(d, act_format, packed_gfx950, x_bf16, T, ldx, router_logits, top_k, renormalize, y_bf16, topk_ids,
                      topk_w, workspace, workspace_bytes, S(stream), events, n_events);
}
