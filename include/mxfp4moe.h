/*
 * mxfp4moe.h -- C ABI of the gfx950 (MI355X) MXFP4 quantization and MXFP4-weight MoE library.
 *
 * Page tags used in the citations below:
 *   [P1] prhub summary of vLLM PR #46915 (weight/scale interleave fix in the SM90 MXFP4 fused-MoE test)
 *   [P2] prhub report of vLLM PR #51038 "[Bugfix][Quantization] Fix MXFP4 conversion for FlashInfer CUTLASS"
 *   [P3] prhub summary of vLLM PR #43557 (E8M0 scale fix in the MXFP4 MoE CUTLASS kernel)
 *   [DEF] definitions this library adopts where the pages name a step without spelling it out: the
 *        OCP Microscaling MXFP4 format (32-element blocks, E2M1 round-to-nearest-even saturating at
 *        +-6, two nibbles per byte), top-k routing over softmax(logits), SwiGLU = silu(w1 half) *
 *        (w3 half), grouped GEMMs and a routing-weighted combine.
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" are HIP device pointers owned by the caller; the library never
 *     allocates, frees or keeps them.  Host pointers ("host") are read during the call only.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  All device work is
 *     enqueued on it; the calls return without synchronizing unless stated otherwise.
 *   - Arguments are validated before any device work; on failure nothing is written and a status
 *     below is returned.  Launch failures return MXFP4_ERR_DEVICE.  NaN/Inf inputs are outside the
 *     contract (no device-side checks).
 *   - Device pointers must be 16-byte aligned unless stated otherwise.
 */
#ifndef MXFP4MOE_H
#define MXFP4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MXFP4_OK = 0,
  MXFP4_ERR_NULL = 1,      /* a required pointer is NULL */
  MXFP4_ERR_SHAPE = 2,     /* a size or dimension is out of range */
  MXFP4_ERR_ALIGN = 3,     /* a pointer or stride breaks the alignment rule */
  MXFP4_ERR_WORKSPACE = 4, /* workspace or output buffer too small */
  MXFP4_ERR_LAYOUT = 5,    /* unknown layout flag, or a packed blob whose header does not match */
  MXFP4_ERR_DEVICE = 6     /* a HIP call or kernel launch failed */
};

/* Static, NUL-terminated description of a status code (unknown codes get a generic string). */
const char* mxfp4_status_str(int status);

/* Library version, (major << 16) | minor. */
uint32_t mxfp4_version(void);

/* ------------------------------------------------------------------------------------------------
 * MXFP4 block quantization.  [P3 Implementation breakdown item 1; Key source snippets: the E8M0
 * reference helper and the UE8M0_SF branch of the FP16/BF16 -> FP4 converter; DEF element rule]
 *
 * For each row of x and each 32-element block along K:
 *   amax = max |x| over the block (bf16 magnitudes, exact);
 *   e    = 0 if amax == 0, else B - 2 clamped to [0, 254], with B the biased exponent of the binary32
 *          bits of amax after adding 2^21 (significands >= 1.75 round up);
 *   code = E2M1 of |x| * 2^(127 - e), round to nearest even, saturating at 6; sign bit 0x8 copied
 *          from x (also when the magnitude code is 0);
 *   q[row][j] = code[2j] | code[2j+1] << 4  (element 2j in the low nibble).
 * x_bf16        device, bf16 [M, ldx] row-major; K % 32 == 0, ldx >= K, ldx % 8 == 0.
 *               Strided (ldx > K) input is read correctly: the pages' linear path had to force a
 *               contiguous copy before quantizing [P3 Implementation breakdown item 2]; here the
 *               stride is explicit.
 * q_u8          device, uint8 [M, K/2], required.
 * scale_flat_u8 device, uint8 [M, K/32], may be NULL; any alignment (byte stores are used unless the
 *               pointer is 4-byte aligned and K/32 is a multiple of 4, then whole dwords).
 * scale_tiled_u8 device, uint8 [ceil(M/128), ceil(K/128), 32, 4, 4], 16-byte aligned (each
 *               [mT][kT][oM] group of 16 bytes is written with one store), may be NULL: the byte at
 *               [mT][kT][oM][iM][iK] is the scale of row mT*128 + iM*32 + oM and scale column
 *               kT*4 + iK; padding bytes are written as 0.  [P3 Key source snippets, the untile
 *               helper's permute (0, 3, 2, 1, 4)]
 * M >= 0 (M == 0 is a no-op), K >= 32.
 */
int mxfp4_quantize(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, void* q_u8, void* scale_flat_u8,
                   void* scale_tiled_u8, void* stream);

/* Bytes of the tiled scale output for an [M, K] matrix: ceil(M/128) * ceil(K/128) * 512. */
size_t mxfp4_tiled_scale_bytes(int64_t M, int64_t K);

/* ------------------------------------------------------------------------------------------------
 * NVFP4 block quantization, the converter's other scale format.  [P3 Implementation breakdown item 1
 * and Key source snippets: the branch taken without UE8M0 scales (max / 6 stored as E4M3, times a
 * global scale); Review highlights item 2: elements are scaled by the dequantized stored scale]
 * For each row of x and each 16-element block along K, in binary32:
 *   SF   = global_scale * (amax * r6), r6 the binary32 nearest to 1/6, amax = max |x| (exact);
 *   s    = SF as E4M3 (round to nearest even; above 448 -> 448), the stored scale byte;
 *   code = E2M1 of |x| * (global_scale / value(s)) (quotient and product rounded to binary32, then
 *          nearest even, saturating at 6; 0 when value(s) is 0), sign bit 0x8 copied from x;
 *   q[row][j] = code[2j] | code[2j+1] << 4.
 * A value decodes as E2M1(code) * value(s) / global_scale.
 * x_bf16 device bf16 [M, ldx]; K % 16 == 0, K >= 16, ldx >= K, ldx % 8 == 0.
 * global_scale: host binary32, positive and finite (else MXFP4_ERR_SHAPE).
 * q_u8 device uint8 [M, K/2], required.  scale_flat_u8 device uint8 [M, K/16], may be NULL, any
 * alignment.  scale_tiled_u8 device, 16-byte aligned, may be NULL: [ceil(M/128), ceil(K/64), 32, 4, 4],
 * the byte at [mT][kT][oM][iM][iK] the scale of row mT*128 + iM*32 + oM and scale column kT*4 + iK
 * (the tiling of mxfp4_quantize over 16-element scale columns), padding bytes 0.
 * M >= 0 (M == 0 is a no-op). */
int nvfp4_quantize(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, float global_scale, void* q_u8,
                   void* scale_flat_u8, void* scale_tiled_u8, void* stream);

/* Bytes of nvfp4_quantize's tiled scale output: ceil(M/128) * ceil(K/64) * 512; 0 for invalid sizes. */
size_t nvfp4_tiled_scale_bytes(int64_t M, int64_t K);

/* ------------------------------------------------------------------------------------------------
 * MoE weight set.  The standard checkpoint layout [P2 Implementation breakdown item 2]:
 *   w13_q uint8 [E, 2I, H/2]  rows [w1 (gate); w3 (up)]     w13_s uint8 [E, 2I, H/32]  E8M0
 *   w2_q  uint8 [E, H, I/2]                                 w2_s  uint8 [E, H, I/32]   E8M0
 *   b13 [E, 2I], b2 [E, H] optional, fp32 or bf16; converted to bf16 (round to nearest even).
 * Requirements: E >= 1, H % 32 == 0, I % 32 == 0, H >= 32, I >= 32.
 */
typedef struct {
  int32_t E, H, I, has_bias;
} mxfp4_moe_dims;

enum {
  MXFP4_LAYOUT_GFX950 = 0,      /* this library's execution layout (opaque blob with a header) */
  MXFP4_LAYOUT_STD_W31 = 1,     /* checked conversion: standard tensors with w13 as [w3; w1] */
  MXFP4_LAYOUT_SCALE_TILED = 2  /* checked conversion flag: scales in the tiled layout above */
};

/* Output bytes of mxfp4_repack_weights for `layout`; 0 for invalid dims or layout. */
size_t mxfp4_repack_bytes(const mxfp4_moe_dims* d, uint32_t layout);

/* Byte offsets of the six tensors inside a checked-conversion output (layout != GFX950), in the
 * order w13_q, w2_q, w13_s, w2_s, b13, b2: the order in which the pages' conversion returns
 * (w13 weight, w2 weight, w13 scale, w2 scale, w13 bias, w2 bias) [P2 Key source snippets, the
 * conversion branch's return tuple and the test's converted[0..5]]; each offset is 256-byte aligned.
 * Returns a status. */
int mxfp4_repack_offsets(const mxfp4_moe_dims* d, uint32_t layout, size_t offsets_out[6]);

/* Weight conversion at load time.  [P2 Implementation breakdown items 1-3, Key source snippets]
 * Inputs are the standard tensors above (device).  b13/b2 are read only when d->has_bias (then
 * required); bias_is_fp32 selects fp32 (else bf16) input, 4-byte/2-byte aligned.
 * layout = MXFP4_LAYOUT_GFX950: writes the execution blob consumed by moe_mxfp4_forward.
 * layout = MXFP4_LAYOUT_STD_W31 [| MXFP4_LAYOUT_SCALE_TILED], or MXFP4_LAYOUT_SCALE_TILED alone:
 *   writes the six standard tensors at mxfp4_repack_offsets() (w13_q, w2_q, w13_s, w2_s, b13, b2 in
 *   that order): w13_q and w13_s with their row halves exchanged ([w1; w3] -> [w3; w1]) when
 *   STD_W31 is set, w2 unchanged, b13 halves exchanged
 *   likewise, both biases as bf16; with SCALE_TILED both scale tensors are written per expert in the
 *   tiled layout [E, ceil(rows/128), ceil(K/128), 32, 4, 4] instead of flat.  These conversions
 *   exist to check this library against the pages' layouts; the forward pass does not use them.
 * Unknown layout bits -> MXFP4_ERR_LAYOUT.  out_bytes < mxfp4_repack_bytes() -> MXFP4_ERR_WORKSPACE.
 */
int mxfp4_repack_weights(const mxfp4_moe_dims* d, const void* w13_q, const void* w13_s, const void* w2_q,
                         const void* w2_s, const void* b13, const void* b2, int32_t bias_is_fp32, uint32_t layout,
                         void* out, size_t out_bytes, void* stream);

/* Inverse of mxfp4_repack_weights(GFX950): writes the standard tensors back (biases as bf16 bit
 * patterns).  Round trip is the identity on q and scales.  Reads the blob header with a
 * synchronous device-to-host copy and returns MXFP4_ERR_LAYOUT if it does not match *d. */
int mxfp4_unpack_weights(const mxfp4_moe_dims* d, const void* packed, void* w13_q, void* w13_s, void* w2_q,
                         void* w2_s, void* b13_bf16, void* b2_bf16, void* stream);

/* Checks a GFX950 blob's header against *d (synchronous device-to-host copy of 256 bytes).
 * MXFP4_OK or MXFP4_ERR_LAYOUT.  moe_mxfp4_forward itself does not read the header. */
int mxfp4_check_packed(const mxfp4_moe_dims* d, const void* packed, void* stream);

/* ------------------------------------------------------------------------------------------------
 * Routing.  [DEF: router logits -> softmax -> top-k, renormalized over the selected experts]
 *   topk_ids[t] = the top_k largest logits of token t in descending order, equal logits in
 *                 increasing expert index (-0.0 equals +0.0);
 *   topk_w[t,j] = exp(l_j - l_max) / S, S summed over the selected experts (renormalize != 0) or
 *                 over all E experts (renormalize == 0), computed in fp32;
 *   expert_offsets [E+1] = exclusive prefix sum of per-expert pair counts;
 *   sorted_pairs [T*top_k]: pairs p = t*top_k + j grouped by expert, increasing p within an expert.
 * router_logits device fp32 [T, E] contiguous; 1 <= top_k <= min(E, 32); 1 <= E <= 1024; T >= 0.
 * Outputs device int32/fp32 (4-byte alignment suffices).  workspace: device,
 * >= moe_mxfp4_route_workspace_bytes(T, E, top_k), 256-byte aligned.
 */
size_t moe_mxfp4_route_workspace_bytes(int64_t T, int32_t E, int32_t top_k);
int moe_mxfp4_route(const float* router_logits, int64_t T, int32_t E, int32_t top_k, int32_t renormalize,
                    int32_t* topk_ids, float* topk_w, int32_t* expert_offsets, int32_t* sorted_pairs, void* workspace,
                    size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------------
 * The MoE layer.  [DEF; P1 Implementation breakdown: the fused-MoE call takes packed 4-bit weights
 * with per-32 group scales and 16-bit activations]
 *   y[t] = sum_j topk_w[t,j] * ( W2_e (silu(h_g) * h_u) + b2_e ),  e = topk_ids[t,j],
 *   h = W13_e x_t + b13_e, h_g = rows [0, I) (w1), h_u = rows [I, 2I) (w3),
 * with W13_e, W2_e the dequantized MXFP4 weights.  Routing as moe_mxfp4_route.
 * packed_gfx950 device blob from mxfp4_repack_weights(GFX950) for the same *d (not re-checked here;
 *   see mxfp4_check_packed).
 * x_bf16  device bf16 [T, ldx], ldx >= H, ldx % 8 == 0.   y_bf16 device bf16 [T, H].
 * router_logits device fp32 [T, E].  topk_ids / topk_w: optional device outputs [T, top_k].
 * workspace device, >= moe_mxfp4_workspace_bytes(d, T, top_k), 256-byte aligned.
 * Size limit: the split activations of the first GEMM (T * H * 2.25 bytes) and of the second (about
 * 2 bytes per padded pair row and I element) must each stay below 4 GiB, else MXFP4_ERR_SHAPE.
 * Arithmetic: activations enter the block-scaled MFMA as three terms with E8M0 scales per 32
 * elements, x = t0 + t1 + t2 (E2M3, E2M3 of the remainder, E2M1 of what is left; each scale from the
 * rule above), weights as E2M1 with their E8M0 scales, fp32 accumulation; the SwiGLU output stays
 * fp32 and is split into three terms the same way; each pair's weighted expert output is kept as
 * integers with a power-of-two scale per 16 columns (at most 2^-14 of the block maximum off), and
 * the combine sums a token's k rows in fp32 in slot order, then rounds to bf16.  The result is
 * deterministic: repeated calls give the same bits.
 */
size_t moe_mxfp4_workspace_bytes(const mxfp4_moe_dims* d, int64_t T, int32_t top_k);

/* Activation formats of moe_mxfp4_forward_act. */
enum {
  MXFP4_ACT_BF16 = 0,  /* bf16 activations, as moe_mxfp4_forward */
  MXFP4_ACT_MXFP8 = 1, /* both GEMM inputs quantized to MXFP8 */
  MXFP4_ACT_MXFP4 = 2  /* both GEMM inputs quantized to MXFP4 */
};
int moe_mxfp4_forward(const mxfp4_moe_dims* d, const void* packed_gfx950, const void* x_bf16, int64_t T, int64_t ldx,
                      const float* router_logits, int32_t top_k, int32_t renormalize, void* y_bf16, int32_t* topk_ids,
                      float* topk_w, void* workspace, size_t workspace_bytes, void* stream);

/* The MoE layer with quantized activations, or bf16 ones (act_format = MXFP4_ACT_BF16 is exactly
 * moe_mxfp4_forward).  [P2 Implementation breakdown item 3: the MXFP8-activation variant of the MXFP4
 * MoE backend; P3 Implementation breakdown item 3: the experts-quant step, MoE activations quantized to
 * MXFP4 with the same E8M0 rule]
 * With MXFP4_ACT_MXFP8 / MXFP4_ACT_MXFP4 the layer input x (each token row, per 32-element block) and
 * the SwiGLU output (fp32, per 32-element block of I) are quantized before the two products and enter
 * the MFMA as one term:
 *   MXFP8: E4M3 elements (round to nearest even) with e = B - 8, B the rounded biased exponent of the
 *          block maximum as in mxfp4_quantize (the pages' rule with E4M3's largest exponent 8 in place
 *          of E2M1's 2), so the maximum maps into [224, 448) and nothing saturates;
 *   MXFP4: exactly the element and scale rule of mxfp4_quantize.
 * Arguments, workspace and errors as moe_mxfp4_forward; an unknown act_format -> MXFP4_ERR_LAYOUT. */
int moe_mxfp4_forward_act(const mxfp4_moe_dims* d, int32_t act_format, const void* packed_gfx950, const void* x_bf16,
                          int64_t T, int64_t ldx, const float* router_logits, int32_t top_k, int32_t renormalize,
                          void* y_bf16, int32_t* topk_ids, float* topk_w, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Same as moe_mxfp4_forward_act, and records events[i] (hipEvent_t passed as void*, created by the caller)
 * on `stream` at stage boundaries: events[0] before the first launch, then after each stage in the
 * order activation split and routing (one launch), pair placement/tile schedule, first GEMM (+SwiGLU),
 * second GEMM (weighted rows), combine (bf16 output) -- 6 events in all.  Only the first n_events are
 * recorded.
 * For per-stage timing (measurement); the computation is identical. */
int moe_mxfp4_forward_profiled(const mxfp4_moe_dims* d, int32_t act_format, const void* packed_gfx950,
                               const void* x_bf16, int64_t T, int64_t ldx, const float* router_logits, int32_t top_k,
                               int32_t renormalize, void* y_bf16, int32_t* topk_ids, float* topk_w, void* workspace,
                               size_t workspace_bytes, void* stream, void* const* events, int32_t n_events);

/* ------------------------------------------------------------------------------------------------
 * Dense MXFP4-weight linear layer (W4A16): y = x W^T + b, W dequantized MXFP4.  [P3 Implementation
 * breakdown item 2: the MXFP4 linear path; DEF: a MoE layer of one expert without routing or
 * activation function]
 * Weights in the standard layout: w_q uint8 [N, K/2] (element 2j in the low nibble), w_s uint8 [N, K/32]
 * E8M0; bias [N] fp32 or bf16 (converted to bf16, round to nearest even), optional.
 * Requirements: N, K multiples of 32, 32 <= N, K <= 2^20.
 * Arithmetic as the second product of moe_mxfp4_forward: x enters as three terms per 32 elements, fp32
 * accumulation, bias added in fp32, one rounding to bf16.
 */
/* Output bytes of mxfp4_linear_pack; 0 for invalid sizes. */
size_t mxfp4_linear_pack_bytes(int64_t N, int64_t K, int32_t has_bias);

/* Weight conversion at load time into this library's layout (opaque, 256-byte header).  w_q, w_s,
 * bias (may be NULL) device; out device, 256-byte aligned, >= mxfp4_linear_pack_bytes (else
 * MXFP4_ERR_WORKSPACE). */
int mxfp4_linear_pack(int64_t N, int64_t K, const void* w_q, const void* w_s, const void* bias, int32_t bias_is_fp32,
                      void* out, size_t out_bytes, void* stream);

/* Workspace bytes of mxfp4_linear_forward for M rows; 0 for invalid sizes. */
size_t mxfp4_linear_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* y_bf16 device bf16 [M, N] (row-major, contiguous, 16-byte aligned) = x_bf16 (device bf16 [M, ldx],
 * ldx >= K, ldx % 8 == 0) times the packed weights (has_bias as packed).  workspace device, 256-byte
 * aligned, >= mxfp4_linear_workspace_bytes(M, N, K).  M == 0 is a no-op; M * K * 2 bytes of split
 * activations must stay below 4 GiB (else MXFP4_ERR_SHAPE).  Deterministic. */
int mxfp4_linear_forward(const void* packed, int64_t N, int64_t K, int32_t has_bias, const void* x_bf16, int64_t M,
                         int64_t ldx, void* y_bf16, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------------
 * The MoE layer without a workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same arguments,
 * arithmetic and result as moe_mxfp4_forward, whose kernels it shares; the workspace is a device
 * array of MXFP4_NOALLOC_SCRATCH_BYTES inside the library (one per device, held until the process
 * ends), so the call allocates nothing.
 * Limit: moe_mxfp4_workspace_bytes(d, T, top_k) must not exceed MXFP4_NOALLOC_SCRATCH_BYTES, else
 *   MXFP4_ERR_WORKSPACE (nothing is launched).  It covers e.g. E = 128, H = 2048, I = 768, top-8 up
 *   to about 200 tokens.
 * The array of the current device is used (make the stream's device current).  Every call on a
 * device shares that device's array: calls that may overlap on one device (streams without ordering
 * between them) race and must not be issued.  Its address is looked up on the first call on each
 * device (MXFP4_ERR_DEVICE if that fails).
 */
#define MXFP4_NOALLOC_SCRATCH_BYTES (32u << 20)
int moe_mxfp4_forward_noalloc(const mxfp4_moe_dims* d, const void* packed_gfx950, const void* x_bf16, int64_t T,
                              int64_t ldx, const float* router_logits, int32_t top_k, int32_t renormalize,
                              void* y_bf16, int32_t* topk_ids, float* topk_w, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4MOE_H */
