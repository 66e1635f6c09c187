// Internal declarations shared by the C-ABI source files: the kernel launchers (each defined next to
// its kernels) and the forward pass's launch sequence (api.cpp), which the entry points call.  Host
// C++ only.
#pragma once

#include <hip/hip_runtime_api.h>

#include "layout.h"

int launch_quantize(const void* x, int64_t M, int64_t K, int64_t ldx, void* q, void* sflat, void* stiled,
                    hipStream_t stream);
int launch_nvfp4_quantize(const void* x, int64_t M, int64_t K, int64_t ldx, float gs, void* q, void* sflat,
                          void* stiled, hipStream_t stream);
int launch_repack_gfx950(const MoeGeom& g, const BlobOffsets& o, bool bias, const void* w13_q, const void* w13_s,
                         const void* w2_q, const void* w2_s, const void* b13, const void* b2, int bias_is_fp32,
                         void* out, hipStream_t stream);
int launch_unpack_gfx950(const MoeGeom& g, const BlobOffsets& o, bool bias, const void* packed, void* w13_q,
                         void* w13_s, void* w2_q, void* w2_s, void* b13, void* b2, hipStream_t stream);
int launch_repack_standard(const MoeGeom& g, bool bias, const void* w13_q, const void* w13_s, const void* w2_q,
                           const void* w2_s, const void* b13, const void* b2, int bias_is_fp32, bool swap, bool tiled,
                           const size_t off[6], void* out, hipStream_t stream);
// The activation split of x into xq (format af) and the routing (ids, weights, per-block expert
// histograms, each pair's rank within its block and expert) in one launch.
int launch_front(int af, const void* x, int64_t T, int64_t ldx, const MoeGeom& g, void* xq, const float* logits, int E,
                 int k, int renormalize, int32_t* ids, float* w, int32_t* blkcnt, int32_t* rank, hipStream_t stream);
int launch_route(const float* logits, int64_t T, int E, int k, int renormalize, int32_t* ids, float* w,
                 int32_t* blkcnt, int32_t* rank, hipStream_t stream);
// pair_prow may be the rank array itself.
int launch_place(const int32_t* ids, const float* w, int32_t* blkcnt, const int32_t* rank, int64_t T, int k, int E,
                 int BM, int BM2, int32_t* offsets, int32_t* poffsets, int32_t* sorted_pairs, int32_t* prow_pair,
                 int32_t* prow_tok, float* prow_w, int32_t* pair_prow, void* tiles, int32_t* ntiles, void* tiles2,
                 int32_t* ntiles2, hipStream_t stream);
int launch_gemm1(int af, int NRG, const GemmArgs& a, int64_t max_tiles, hipStream_t stream);
int launch_gemm2(int af, int NRG, const GemmArgs& a, int64_t max_tiles, hipStream_t stream);
int launch_gemm1_mx(int af, int NRG, const GemmArgs& a, int64_t max_tiles, hipStream_t stream);
int launch_gemm2_mx(int af, int NRG, const GemmArgs& a, int64_t max_tiles, hipStream_t stream);
int launch_pack_linear(const MoeGeom& g, const LinearOffsets& o, bool bias, const void* w_q, const void* w_s,
                       const void* b, int bias_is_fp32, void* out, hipStream_t stream);
int launch_linear_prep(const void* x, int64_t M, int64_t ldx, const MoeGeom& g, const LinearWs& w, uint8_t* ws,
                       hipStream_t stream);
int launch_combine(const uint16_t* o16, const uint8_t* osc, const int32_t* pair_prow, void* y, int64_t T, int64_t H, int k,
                   hipStream_t stream);

// The MoE forward pass on a caller-given workspace: argument validation, then the launches in stream
// order; events (may be NULL) are recorded at the stage boundaries.  Returns a status.
int forward_impl(const mxfp4_moe_dims* d, int32_t act_format, const void* packed_gfx950, const void* x_bf16,
                 int64_t T, int64_t ldx, const float* router_logits, int32_t top_k, int32_t renormalize, void* y_bf16,
                 int32_t* topk_ids, float* topk_w, void* workspace, size_t workspace_bytes, hipStream_t s,
                 void* const* events, int32_t n_events);
