// Host-visible layouts of the gfx950 MXFP4 / MoE library: the execution blob of the MoE weights, the
// forward pass's workspace, and the argument records of the kernels.  Plain C++ (no device code), so
// the argument validation that uses it also builds with a host compiler.
#pragma once

#include <stdint.h>

#include "../../include/mxfp4moe.h"

// ---------------------------------------------------------------------------------------------
// Execution layout of the MoE weights (the blob written by mxfp4_repack_weights(GFX950)).
//
// The GEMMs run on v_mfma_scale_f32_32x32x64_f8f6f4.  For an operand tile of 32 rows x 64 K, lane l
// holds row (l % 32) and the 32 consecutive K of block (l / 32); fp4 is 16 bytes per lane (element
// i in nibble i, low nibble first), fp6 is 24 bytes per lane (element i in bits 6i..6i+5); the lane's
// E8M0 scale is one byte of a 32-bit register selected by the instruction's op_sel.
//
// Weight tiles (32 output rows each) are grouped in column blocks of kCB = 16 tiles.  Per expert, per
// column block and per 64-wide K step the blob holds the 16 tiles' operands back to back (16 KB, one
// 1 KB piece per tile in lane order) and then, in the scale array, one 16-byte record per lane with
// the scale byte of each of the 16 tiles:
//   w13 q : [E][ncb1][nkt1][16 tiles][64 lanes][16 B]   tile j of block c: activation tile
//           it = 8c + j/2, gate (w1 rows it*32..) for even j, up (w3 rows) for odd j; lane l: row
//           l%32 of the tile, K block 2*kt + l/32 along H.  Tiles past I/32 and blocks past H/32 are 0.
//   w13 s : [E][ncb1][nkt1][64 lanes][16 tiles]  bytes
//   w2 q  : [E][ncb2][nkt2][16][64][16 B]   tile j of block c: output columns (16c + j)*32.. of H;
//           lane l: row l%32 of the tile, K block 2*kt + l/32 along I, elements of the block in the
//           order W2_PERM (the order in which the first GEMM's epilogue leaves the activation).
//   w2 s  : [E][ncb2][nkt2][64][16]
//   b13   : bf16 [E][2I] (gate half first), b2 : bf16 [E][H]
// nkt = ceil(K / 64) steps along K; ncb1 = ceil(2 * (I/32) / 16), ncb2 = ceil((H/32) / 16).
struct BlobHeader {
  char magic[8];
  uint32_t version;
  int32_t E, H, I, has_bias;
  uint32_t reserved0;
  uint64_t off_w13q, off_w13s, off_w2q, off_w2s, off_b13, off_b2, total;
};
static_assert(sizeof(BlobHeader) <= 256, "header fits in 256 bytes");

#define MX_BLOB_MAGIC "MX4GFX95"
#define MX_BLOB_VERSION 2u

constexpr int kCB = 16;  // weight tiles per column block

struct MoeGeom {
  int64_t E, H, I;
  int64_t nkt1, nkt2;  // 64-wide K steps along H (first GEMM) and along I (second GEMM)
  int64_t nit, nht;    // I/32, H/32
  int64_t ncb1, ncb2;  // column blocks of the two GEMMs
};

static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
static inline int64_t align256(int64_t a) { return (a + 255) & ~(int64_t)255; }

static inline MoeGeom moe_geom(int64_t E, int64_t H, int64_t I) {
  MoeGeom g;
  g.E = E; g.H = H; g.I = I;
  g.nkt1 = cdiv(H, 64);
  g.nkt2 = cdiv(I, 64);
  g.nit = I / 32; g.nht = H / 32;
  g.ncb1 = cdiv(2 * g.nit, kCB);
  g.ncb2 = cdiv(g.nht, kCB);
  return g;
}

struct BlobOffsets {
  uint64_t w13q, w13s, w2q, w2s, b13, b2, total;
};

static inline BlobOffsets blob_offsets(const MoeGeom& g, bool bias) {
  BlobOffsets o;
  uint64_t p = 256;
  o.w13q = p; p = align256(p + (uint64_t)g.E * g.ncb1 * g.nkt1 * kCB * 1024);
  o.w13s = p; p = align256(p + (uint64_t)g.E * g.ncb1 * g.nkt1 * 1024);
  o.w2q = p;  p = align256(p + (uint64_t)g.E * g.ncb2 * g.nkt2 * kCB * 1024);
  o.w2s = p;  p = align256(p + (uint64_t)g.E * g.ncb2 * g.nkt2 * 1024);
  o.b13 = p;  p = align256(p + (bias ? (uint64_t)g.E * 2 * g.I * 2 : 0));
  o.b2 = p;   p = align256(p + (bias ? (uint64_t)g.E * g.H * 2 : 0));
  o.total = p;
  return o;
}

// ---------------------------------------------------------------------------------------------
// Activation formats of the layer (MXFP4_ACT_* in the public header): the format in which both GEMMs
// take their token operand (the layer input, then the SwiGLU output).  The MFMA's B operand is one or
// more terms per 32-element block, each with its own E8M0 scale byte:
//   kActBf16:  bf16-accurate activations as three terms v = t0 + t1 + t2 -- E2M3 (FP6), E2M3 of the
//              remainder, E2M1 (FP4) of what is left -- each scale from the 0.75 round-up rule;
//              24 + 24 + 16 bytes per lane
//   kActMxfp8: one E4M3 (FP8) term, scale rule for E4M3 elements (block maximum to [224, 448)); 32 bytes
//   kActMxfp4: one E2M1 term, the weights' rule; 16 bytes
// A lane's terms sit back to back in one slot; the scale bytes of a slot in one dword (term t in byte
// t, the other bytes zero).
enum : int { kActBf16 = 0, kActMxfp8 = 1, kActMxfp4 = 2 };
constexpr int kFmtFp8 = 0, kFmtFp6 = 2, kFmtFp4 = 4;  // MFMA operand format codes (E4M3, E2M3, E2M1)

constexpr int act_terms(int af) { return af == kActBf16 ? 3 : 1; }
constexpr int act_term_fmt(int af, int t) {
  return af == kActMxfp8 ? kFmtFp8 : af == kActMxfp4 ? kFmtFp4 : (t < 2 ? kFmtFp6 : kFmtFp4);
}
constexpr int fmt_bytes(int fmt) { return fmt == kFmtFp8 ? 32 : fmt == kFmtFp6 ? 24 : 16; }
constexpr int act_term_offset(int af, int t) {
  return t == 0 ? 0 : act_term_offset(af, t - 1) + fmt_bytes(act_term_fmt(af, t - 1));
}
constexpr int act_slot(int af) { return act_term_offset(af, act_terms(af)); }
// The slots of one row group and K step (64 lanes) are stored region by region: a slot's bytes are cut
// where the second GEMM's LDS loads cut them (an E2M3 term into 16 + 8 bytes at a 16-byte boundary or
// 8 + 16 after one, E4M3 into two 16-byte halves, E2M1 whole), and region [o, o + n) of slot L sits at
// 64 * o + n * L.  A wave's load of one region then reads consecutive bytes, free of LDS bank conflicts,
// where lanes reading one slot each at the slot stride would collide.
constexpr int slot_region_start(int af, int o) {
  for (int t = 0; t < act_terms(af); t++) {
    const int off = act_term_offset(af, t), nb = fmt_bytes(act_term_fmt(af, t));
    if (o >= off && o < off + nb) {
      const int first = nb == 24 ? (off % 16 == 0 ? 16 : 8) : 16;
      return o < off + first ? off : off + first;
    }
  }
  return -1;
}
constexpr int slot_region_bytes(int af, int o) {
  const int st = slot_region_start(af, o);
  int end = st + 1;
  while (end < act_slot(af) && slot_region_start(af, end) == st) end++;
  return end - st;
}
// Byte offset of slot byte o of lane L within its row group's and K step's 64 * act_slot(af) bytes.
constexpr int slot_byte(int af, int L, int o) {
  return 64 * slot_region_start(af, o) + slot_region_bytes(af, o) * L + (o - slot_region_start(af, o));
}
static_assert(slot_region_bytes(kActBf16, 0) == 16 && slot_region_bytes(kActBf16, 16) == 8 &&
                  slot_region_bytes(kActBf16, 24) == 8 && slot_region_bytes(kActBf16, 32) == 16 &&
                  slot_region_bytes(kActBf16, 48) == 16 && slot_region_bytes(kActMxfp8, 16) == 16 &&
                  slot_region_bytes(kActMxfp4, 0) == 16,
              "slot regions");
// The first GEMM's activation record of one token and one 64-wide K step: the two blocks' slots, their
// two scale dwords, 8 zero bytes (144, 80 or 48 bytes); records of a token row are consecutive, so the
// first GEMM copies a row's terms and scales together in 16-byte chunks.
constexpr int act_rec(int af) { return 2 * act_slot(af) + 16; }
constexpr int kMaxSlot = 64, kMaxRec = 144;  // the largest format (kActBf16), for workspace sizes
static_assert(act_slot(kActBf16) == kMaxSlot && act_rec(kActBf16) == kMaxRec, "largest format");
static_assert(act_slot(kActMxfp8) == 32 && act_slot(kActMxfp4) == 16, "slot sizes");

// ---------------------------------------------------------------------------------------------
// Forward-pass workspace.  Rows of the expert-sorted order are padded per expert to a multiple of
// 32 ("padded rows"); a padded row with no pair has pair index -1, token 0 and weight 0.
//   blkcnt : [nblk_route][E]  pairs per (block of kRouteTokens tokens, expert); after the scan, the
//            exclusive prefix over blocks
//   xq  : [T][nkt1][act_rec]  per token and K step of x: the two 32-element blocks' slots (terms of the
//         activation format), then per block the dword of its scale bytes, then 8 zero bytes
//   actq: [row group of 32][nkt2][64 lanes][act_slot]  the second GEMM's activation operand, lane
//         (row l%32, K block l/32)
//   acts: [row group][nkt2][64 lanes][4]  the matching scale dwords
//   (sized for the largest format; the other formats use the front of each buffer)
//   tiles, tiles2: TileDesc (expert, first padded row, valid rows, 0) per M tile of the first and of the
//         second GEMM (their tile heights may differ)
//   pair_prow: [T*k] padded row of each (token, slot) pair (until the placement writes it: the pair's rank
//            among its expert's pairs within its token block, from the routing)
//   o16 : int16 [padded rows][H], row r = w * (expert output + b2) of the pair at row r, divided by
//         the power of two 2^(osc - 127) of its block and rounded to an integer (|value| < 2^14)
//   osc : [padded rows][H / 16] bytes, the block exponents: one per 16 consecutive columns of a row
constexpr int kRouteTokens = 64;

struct FwdWs {
  uint64_t blkcnt, offsets, poffsets, sorted_pairs, ids, w, prow_pair, prow_tok, prow_w, pair_prow, tiles, ntiles, tiles2,
      ntiles2, xq, actq, acts, o16, osc, total;
  int64_t nrows_alloc, max_tiles;
};

static inline FwdWs fwd_ws(const MoeGeom& g, int64_t T, int64_t k) {
  FwdWs w;
  const int64_t P = T * k;
  w.nrows_alloc = ((P + 31 * g.E + 31) / 32) * 32 + 128;
  w.max_tiles = cdiv(P, 32) + g.E;
  uint64_t p = 0;
  auto take = [&](uint64_t bytes) { uint64_t o = p; p = align256(p + bytes); return o; };
  w.blkcnt = take(4 * cdiv(T, kRouteTokens) * g.E);
  w.offsets = take(4 * (g.E + 1));
  w.poffsets = take(4 * (g.E + 1));
  w.sorted_pairs = take(4 * P);
  w.ids = take(4 * P);
  w.w = take(4 * P);
  w.prow_pair = take(4 * w.nrows_alloc);
  w.prow_tok = take(4 * w.nrows_alloc);
  w.prow_w = take(4 * w.nrows_alloc);
  w.pair_prow = take(4 * P);
  w.tiles = take(16 * w.max_tiles);
  w.ntiles = take(16);
  w.tiles2 = take(16 * w.max_tiles);
  w.ntiles2 = take(16);
  w.xq = take((uint64_t)T * g.nkt1 * kMaxRec);
  w.actq = take((uint64_t)(w.nrows_alloc / 32) * g.nkt2 * 64 * kMaxSlot);
  w.acts = take((uint64_t)(w.nrows_alloc / 32) * g.nkt2 * 64 * 4);
  w.o16 = take((uint64_t)w.nrows_alloc * g.H * 2);
  w.osc = take((uint64_t)w.nrows_alloc * (g.H / 16));
  w.total = p;
  return w;
}

// One M tile of a grouped GEMM: its expert, first padded row and number of valid rows (one 16-byte load).
struct alignas(16) TileDesc {
  int32_t e, prow0, nrows, pad;
};

// Execution layout of a dense MXFP4 linear layer y = x W^T + b (mxfp4_linear_pack): a 256-byte header,
// then W [N, K] in the second GEMM's layout for one expert with H = N output rows and I = K (pieces
// [ncb2][nkt2][16 tiles][64 lanes][16 B], block elements in w2_perm order; scale records
// [ncb2][nkt2][64][16]), then the bias as bf16 [N] if present.
#define MX_LINEAR_MAGIC "MX4LIN95"

struct LinearOffsets {
  uint64_t wq, ws, bias, total;
};

static inline LinearOffsets linear_offsets(const MoeGeom& g, bool bias) {
  LinearOffsets o;
  uint64_t p = 256;
  o.wq = p;   p = align256(p + (uint64_t)g.ncb2 * g.nkt2 * kCB * 1024);
  o.ws = p;   p = align256(p + (uint64_t)g.ncb2 * g.nkt2 * 1024);
  o.bias = p; p = align256(p + (bias ? (uint64_t)g.H * 2 : 0));
  o.total = p;
  return o;
}

// Linear-layer workspace: the activation operand in the second GEMM's layout (row groups of 32 rows;
// kActBf16 terms in w2_perm order) and its scale dwords, the M tiles of 32 rows, their count, and a
// unit weight per row (plus 64 slack entries read by the row-table copies).
struct LinearWs {
  uint64_t actq, acts, tiles, ntiles, roww, total;
  int64_t nrg;
};

static inline LinearWs linear_ws(int64_t M, const MoeGeom& g) {
  LinearWs w;
  w.nrg = cdiv(M, 32);
  uint64_t p = 0;
  auto take = [&](uint64_t bytes) { uint64_t o = p; p = align256(p + bytes); return o; };
  w.actq = take((uint64_t)w.nrg * g.nkt2 * 64 * kMaxSlot);
  w.acts = take((uint64_t)w.nrg * g.nkt2 * 64 * 4);
  w.tiles = take(16 * (uint64_t)w.nrg);
  w.ntiles = take(16);
  w.roww = take(4 * ((uint64_t)w.nrg * 32 + 64));
  w.total = p;
  return w;
}

// Arguments of the grouped GEMM kernels (device pointers into the blob and the workspace, and the
// 32-bit sizes the kernels index with).
struct GemmArgs {
  const uint8_t* wq;        // weight pieces of this GEMM
  const uint8_t* ws;        // weight scale records
  const uint16_t* bias;     // b13 or b2 (bf16) or NULL
  const uint8_t* xq;        // first GEMM: per-token K-step records; second: activation slots by row group
  const uint8_t* xs;        // second GEMM: matching scale dwords (the first GEMM's are in its records)
  const int32_t* prow_tok;  // padded row -> token
  const int32_t* prow_pair; // padded row -> pair (-1 = padding)
  const float* prow_w;      // padded row -> routing weight
  const TileDesc* tiles;
  const int32_t* ntiles;
  uint8_t* actq;            // first GEMM output
  uint8_t* acts;
  uint16_t* ydense;         // second GEMM in a dense linear layer: bf16 rows [rows][H] (else NULL)
  uint16_t* o16;            // second GEMM output (int16 blocks, padded-row order) and their exponents
  uint8_t* osc;
  int32_t nkt, ncb;         // K steps and column blocks of this GEMM
  int32_t ntl;              // output column tiles of this GEMM (I/32 activation tiles, or H/32)
  int32_t nkt2;             // K steps of the second GEMM (layout of the activation)
  int32_t nrec;             // records per token row of xq (K steps of the first GEMM)
  int32_t I, H;
};
