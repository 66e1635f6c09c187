// MXFP4 block quantization of a bf16 matrix on gfx950.
//
// [P3 Implementation breakdown item 1; Key source snippets: the E8M0 reference helper, the UE8M0_SF
//  branch of the FP16/BF16 -> FP4 converter and the tiled-scale untile helper; DEF element rule]
//
// Work split: a wave covers 512 consecutive columns (16 blocks) of four rows 32 apart, rows
// mT*128 + iM*32 + oM for iM = 0..3 (a workgroup's four waves take four consecutive oM); lane l owns
// eight bf16 (one 16-byte load) of each row, four lanes per 32-element block.  The four rows are the
// four iM of one 16-byte group of the tiled scale layout, so each group is written whole, by one lane
// with one store.  The block maximum is a
// max of bf16 magnitude bits (monotone for non-negative values), reduced over the four lanes.
// Cross-lane steps are DPP moves (no LDS round trips).  Elements are encoded by v_cvt_scalef32_pk_fp4_bf16, which divides by the E8M0 scale and rounds
// to nearest even with saturation and a kept sign -- the element rule exactly (checked against the
// oracle on every bf16 pattern under every exponent).  The grid also covers the padding of the tiled
// layout (rows up to a multiple of 128, columns up to a multiple of 128), whose lanes read nothing and
// write zero scale bytes there.
#include "common.h"
#include "internal.h"

namespace {

constexpr int kRowsPerWave = 4;
constexpr int kWaves = 4;
constexpr int kRowsPerBlock = kRowsPerWave * kWaves;  // 16

__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                       int64_t ldx, uint8_t* __restrict__ q,
                                                       uint8_t* __restrict__ sflat, uint8_t* __restrict__ stiled,
                                                       int64_t Mpad, int64_t Kpad, int64_t kTiles,
                                                       bool flat_words) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t col = (int64_t)blockIdx.x * 512 + lane * 8;
  const bool col_live = col < Kpad;   // uniform over each 16-lane (128-column) group
  const bool col_in = col < K;        // uniform over each 4-lane block (K % 32 == 0)
  const int64_t nby = Mpad / kRowsPerBlock;
  for (int64_t by = blockIdx.y; by < nby; by += gridDim.y) {
  // row r of this wave: mT * 128 + r * 32 + oM (128 / kRowsPerBlock = 8 workgroups per 128-row tile)
  const int64_t mT = by >> 3, oM = ((by & 7) << 2) + wave;
  const int64_t row0 = mT * 128 + oM;
  uint32_t tw[kRowsPerWave];  // tiled scale words of the four rows (lanes 16j)

  u32x4_t v[kRowsPerWave];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; r++) {
    const int64_t row = row0 + 32 * r;
    if (col_in && row < M)
      v[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(x + row * ldx + col));
    else
      v[r] = u32x4_t{0u, 0u, 0u, 0u};
  }

#pragma unroll
  for (int r = 0; r < kRowsPerWave; r++) {
    const int64_t row = row0 + 32 * r;
    // largest magnitude among this lane's eight values
    uint32_t w[4] = {v[r][0], v[r][1], v[r][2], v[r][3]};
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      uint32_t lo = w[i] & 0x7FFFu, hi = (w[i] >> 16) & 0x7FFFu;
      m = max(m, max(lo, hi));
    }
    // maximum over the block's four lanes (DPP quad permutations: lane ^ 1, lane ^ 2)
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false));
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, false));
    const uint32_t e = e8m0_from_amax_bits(m << 16);
    const float s = e8m0_as_scale_operand(e);

    uint32_t packed = 0;
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, __builtin_bit_cast(bf16x2_t, w[0]), s, 0);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, __builtin_bit_cast(bf16x2_t, w[1]), s, 1);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, __builtin_bit_cast(bf16x2_t, w[2]), s, 2);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, __builtin_bit_cast(bf16x2_t, w[3]), s, 3);

    // the scales of the four blocks of a 128-column group live in lanes 16j, 16j+4, 16j+8, 16j+12
    // (DPP rotations within each 16-lane row bring lanes +4, +8, +12 to lane 16j): one dword for the
    // tiled layout and, where the row's flat scales are dword-aligned and the group lies inside K, for
    // the flat layout too
    const uint32_t e1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)e, 0x12C, 0xF, 0xF, false);
    const uint32_t e2 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)e, 0x128, 0xF, 0xF, false);
    const uint32_t e3 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)e, 0x124, 0xF, 0xF, false);
    const uint32_t word = e | (e1 << 8) | (e2 << 16) | (e3 << 24);
    const bool live = col_in && row < M;
    if (live) {
      // nibbles are written once and not read again here: streaming stores
      __builtin_nontemporal_store(packed, reinterpret_cast<uint32_t*>(q + row * (K / 2) + col / 2));
      if (sflat) {
        if (flat_words && col + 128 <= K) {
          if ((lane & 15) == 0) *reinterpret_cast<uint32_t*>(sflat + row * (K / 32) + col / 32) = word;
        } else if ((lane & 3) == 0) {
          sflat[row * (K / 32) + col / 32] = (uint8_t)e;
        }
      }
    }
    tw[r] = word;
  }
  // the 16-byte tiled group (mT, kT, oM): the words of iM = 0..3
  if (stiled && col_live && (lane & 15) == 0) {
    const int64_t kT = col >> 7;
    *reinterpret_cast<u32x4_t*>(stiled + ((mT * kTiles + kT) * 32 + oM) * 16) = u32x4_t{tw[0], tw[1], tw[2], tw[3]};
  }
  }
}

// ------------------------------------------------------------------------------------------------
// NVFP4: the converter's non-E8M0 branch.  [P3 Key source snippets, the NVFP4 branch of the
// FP16/BF16 -> FP4 converter; Review highlights item 2, elements scaled by the dequantized scale]
// Per 16-element block, in binary32: SF = gs * (max|x| * fl(1/6)); the stored byte is SF as E4M3
// (nearest even; SF above 448 saturates); SF_deq = its value; r = gs / SF_deq (0 when SF_deq is 0);
// element code = E2M1 of x * r (nearest even, saturating at 6, sign kept).  Same work split as the MXFP4
// kernel: a wave covers 512 columns of four rows 32 apart, lane l owns eight bf16 (half a block, two
// lanes per block); the four scale bytes of one 64-column group of the tiled layout sit in lanes 8j,
// 8j + 2, 8j + 4, 8j + 6 and DPP row shifts bring them to lane 8j, which writes the group.
typedef short q_s16x2_t __attribute__((ext_vector_type(2)));
constexpr float kRcp6 = 0x1.555556p-3f;  // the binary32 nearest to 1/6

__global__ __launch_bounds__(256) void nvfp4_quantize_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                             int64_t ldx, float gs, uint8_t* __restrict__ q,
                                                             uint8_t* __restrict__ sflat, uint8_t* __restrict__ stiled,
                                                             int64_t Mpad, int64_t Kpad, int64_t kTiles,
                                                             bool flat_words) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t col = (int64_t)blockIdx.x * 512 + lane * 8;
  const bool col_live = col < Kpad;  // uniform over each 8-lane (64-column) group
  const bool col_in = col < K;       // uniform over each 2-lane block (K % 16 == 0)
  const int64_t nby = Mpad / kRowsPerBlock;
  for (int64_t by = blockIdx.y; by < nby; by += gridDim.y) {
    const int64_t mT = by >> 3, oM = ((by & 7) << 2) + wave;
    const int64_t row0 = mT * 128 + oM;
    uint32_t tw[kRowsPerWave];
    u32x4_t v[kRowsPerWave];
#pragma unroll
    for (int r = 0; r < kRowsPerWave; r++) {
      const int64_t row = row0 + 32 * r;
      if (col_in && row < M)
        v[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(x + row * ldx + col));
      else
        v[r] = u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int r = 0; r < kRowsPerWave; r++) {
      const int64_t row = row0 + 32 * r;
      const uint32_t w[4] = {v[r][0], v[r][1], v[r][2], v[r][3]};
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < 4; i++) m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
      m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false));  // lane ^ 1
      const float vmax = bf16_bits_to_f32(m);
      const float sf = gs * (vmax * kRcp6);
      q_s16x2_t sb = q_s16x2_t{0, 0};
      sb = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(sb, fminf(sf, 448.0f), 0.0f, 1.0f, false);
      const uint32_t e = (uint32_t)__builtin_bit_cast(uint32_t, sb) & 0xFFu;
      const float sf_deq = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(e, 1.0f, false)[0];
      const float rs = sf_deq > 0.0f ? gs / sf_deq : 0.0f;
      float sv[8];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        sv[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu) * rs;
        sv[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16) * rs;
      }
      uint32_t packed = 0;
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, sv[0], sv[1], 1.0f, 0);
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, sv[2], sv[3], 1.0f, 1);
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, sv[4], sv[5], 1.0f, 2);
      packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, sv[6], sv[7], 1.0f, 3);
      // the scale bytes of the group's four blocks: lanes 8j, 8j + 2, 8j + 4, 8j + 6 (row_shl 2, 4, 6)
      const uint32_t e1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)e, 0x102, 0xF, 0xF, false);
      const uint32_t e2 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)e, 0x104, 0xF, 0xF, false);
      const uint32_t e3 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)e, 0x106, 0xF, 0xF, false);
      const uint32_t word = e | (e1 << 8) | (e2 << 16) | (e3 << 24);
      if (col_in && row < M) {
        __builtin_nontemporal_store(packed, reinterpret_cast<uint32_t*>(q + row * (K / 2) + col / 2));
        if (sflat) {
          if (flat_words && col + 64 <= K) {
            if ((lane & 7) == 0) *reinterpret_cast<uint32_t*>(sflat + row * (K / 16) + col / 16) = word;
          } else if ((lane & 1) == 0) {
            sflat[row * (K / 16) + col / 16] = (uint8_t)e;
          }
        }
      }
      tw[r] = word;
    }
    if (stiled && col_live && (lane & 7) == 0) {
      const int64_t kT = col >> 6;
      *reinterpret_cast<u32x4_t*>(stiled + ((mT * kTiles + kT) * 32 + oM) * 16) = u32x4_t{tw[0], tw[1], tw[2], tw[3]};
    }
  }
}

}  // namespace

int launch_nvfp4_quantize(const void* x, int64_t M, int64_t K, int64_t ldx, float gs, void* q, void* sflat,
                          void* stiled, hipStream_t stream) {
  const int64_t mTiles = (M + 127) / 128;
  const int64_t kTiles = (K / 16 + 3) / 4;
  const int64_t Mpad = mTiles * 128;
  const int64_t Kpad = kTiles * 64;
  const int64_t nby = Mpad / kRowsPerBlock;
  dim3 grid((unsigned)((Kpad + 511) / 512), (unsigned)(nby < 65535 ? nby : 65535));
  const bool flat_words = (K / 16) % 4 == 0 && ((uintptr_t)sflat & 3u) == 0;
  hipLaunchKernelGGL(nvfp4_quantize_kernel, grid, dim3(256), 0, stream, (const uint16_t*)x, M, K, ldx, gs, (uint8_t*)q,
                     (uint8_t*)sflat, (uint8_t*)stiled, Mpad, Kpad, kTiles, flat_words);
  return hipGetLastError() == hipSuccess ? MXFP4_OK : MXFP4_ERR_DEVICE;
}

int launch_quantize(const void* x, int64_t M, int64_t K, int64_t ldx, void* q, void* sflat, void* stiled,
                    hipStream_t stream) {
  const int64_t mTiles = (M + 127) / 128;
  const int64_t kTiles = (K / 32 + 3) / 4;
  const int64_t Mpad = mTiles * 128;
  const int64_t Kpad = kTiles * 128;
  const int64_t nby = Mpad / kRowsPerBlock;
  dim3 grid((unsigned)((Kpad + 511) / 512), (unsigned)(nby < 65535 ? nby : 65535));
  // flat scales as whole dwords only where every row's scales start on a dword boundary (the flat
  // output itself needs only byte alignment)
  const bool flat_words = (K / 32) % 4 == 0 && ((uintptr_t)sflat & 3u) == 0;
  hipLaunchKernelGGL(quantize_kernel, grid, dim3(256), 0, stream, (const uint16_t*)x, M, K, ldx, (uint8_t*)q,
                     (uint8_t*)sflat, (uint8_t*)stiled, Mpad, Kpad, kTiles, flat_words);
  return hipGetLastError() == hipSuccess ? MXFP4_OK : MXFP4_ERR_DEVICE;
}
