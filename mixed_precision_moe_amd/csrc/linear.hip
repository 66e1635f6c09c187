// The dense MXFP4-weight linear layer y = x W^T + b: the activation split of x's rows into the second
// grouped GEMM's operand layout, which that GEMM (one expert, N output rows, K reduction) then
// multiplies with a dense bf16 epilogue.
//
// [P3 Implementation breakdown item 2: the MXFP4 linear path; DEF: W4A16 linear layer, a MoE layer of
//  one expert without routing or activation function]
//
// linear_prep_kernel: one thread per (row, 32-element block), rows padded to a multiple of 32 and
// blocks to whole 64-wide K steps with zeros.  The block's elements are put in w2_perm order (the
// order of the packed weights' blocks), split into the three terms of kActBf16 (E2M3, E2M3 of the
// remainder, E2M1 of what is left, scales from the 0.75 round-up rule) and written as the operand slot
// of lane (block % 2) * 32 + row % 32 of K step block / 2 of the row group.  Threads are ordered row
// fastest within a row group, so consecutive threads write consecutive slots.  The kernel also writes
// the M-tile list (32-row tiles of the single expert) and unit row weights.
#include "common.h"
#include "internal.h"

namespace {

__global__ __launch_bounds__(256) void linear_prep_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                          int64_t ldx, int64_t nkt, int64_t nrg,
                                                          uint8_t* __restrict__ actq, uint32_t* __restrict__ acts,
                                                          TileDesc* __restrict__ tiles, int32_t* __restrict__ ntiles,
                                                          float* __restrict__ roww) {
  constexpr int SLOT = act_slot(kActBf16);
  const int64_t nb2 = 2 * nkt;  // blocks per row, padded to whole K steps
  const int64_t n = nrg * nb2 * 32;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < nrg * 32 + 64; j += stride) {
    roww[j] = 1.0f;
    if (j < nrg) tiles[j] = TileDesc{0, (int32_t)(32 * j), (int32_t)min((int64_t)32, M - 32 * j), 0};
    if (j == 0) *ntiles = (int32_t)nrg;
  }
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int64_t rlo = i % 32, b = (i / 32) % nb2, rg = i / (32 * nb2);
    const int64_t row = rg * 32 + rlo;
    uint32_t src[16];
    if (row < M && b < K / 32) {
      const u32x4_t* p = reinterpret_cast<const u32x4_t*>(x + row * ldx + b * 32);
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const u32x4_t v = __builtin_nontemporal_load(p + q);
        src[4 * q] = v[0]; src[4 * q + 1] = v[1]; src[4 * q + 2] = v[2]; src[4 * q + 3] = v[3];
      }
    } else {
#pragma unroll
      for (int q = 0; q < 16; q++) src[q] = 0u;
    }
    // position p holds element w2_perm(p); pairs (2j, 2j + 1) stay together, so whole words move
    uint32_t w[16];
#pragma unroll
    for (int j = 0; j < 16; j++) w[j] = src[w2_perm(2 * j) / 2];
    uint32_t slot[SLOT / 4];
    const uint32_t scales = split3_bf16(w, slot);
    const int64_t blk = rg * nkt + b / 2;
    const int L = (int)((b & 1) * 32 + rlo);
    store_slot<kActBf16>(actq + blk * 64 * SLOT, L, slot);
    acts[blk * 64 + L] = scales;
  }
}

}  // namespace

int launch_linear_prep(const void* x, int64_t M, int64_t ldx, const MoeGeom& g, const LinearWs& w, uint8_t* ws,
                       hipStream_t stream) {
  const int64_t n = w.nrg * 2 * g.nkt2 * 32;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(linear_prep_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const uint16_t*)x, M, g.I, ldx,
                     g.nkt2, w.nrg, ws + w.actq, (uint32_t*)(ws + w.acts), (TileDesc*)(ws + w.tiles),
                     (int32_t*)(ws + w.ntiles), (float*)(ws + w.roww));
  return hipGetLastError() == hipSuccess ? MXFP4_OK : MXFP4_ERR_DEVICE;
}
