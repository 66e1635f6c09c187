// The bf16-activation instantiations of the grouped GEMM kernels (gemm_kernel.h), the launch
// dispatch over activation formats, and the final combine over the top-k experts of each token.
#include "gemm_kernel.h"

namespace {

// y[t] = sum over the token's k pairs of the int16 rows (times their block powers of two), fp32 sum in
// slot order, bf16 output.  One thread per 8 output columns of a token; the rows of eight (then four)
// pairs are loaded before any is added, so that many gathers per thread are in flight.
MX_DEV void combine_add(float* s, const u32x4_t& v, int ex) {
  const float f = __builtin_ldexpf(1.0f, ex);  // exact power of two (ex in [-127, 127])
#pragma unroll
  for (int q = 0; q < 8; q++) {
    const int16_t hb = (int16_t)(uint16_t)(v[q >> 1] >> (16 * (q & 1)));
    s[q] += (float)hb * f;  // |hb| < 2^14: exact in fp32, as is the product by a power of two
  }
}

__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ o16, const uint8_t* __restrict__ osc,
                                                      const int32_t* __restrict__ pair_prow, uint16_t* __restrict__ y,
                                                      int64_t H, int k, int64_t n) {
  const int64_t H8 = H / 8;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / H8, c = (i - t * H8) * 8;
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int j = 0;
    for (; j + 8 <= k; j += 8) {
      u32x4_t v[8];
      int ex[8];
#pragma unroll
      for (int u = 0; u < 8; u++) {
        const int64_t r = pair_prow[t * k + j + u];
        v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(o16 + r * H + c));
        ex[u] = (int)osc[r * (H / 16) + c / 16] - 127;
      }
#pragma unroll
      for (int u = 0; u < 8; u++) combine_add(s, v[u], ex[u]);
    }
    for (; j + 4 <= k; j += 4) {
      u32x4_t v[4];
      int ex[4];
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const int64_t r = pair_prow[t * k + j + u];
        v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(o16 + r * H + c));
        ex[u] = (int)osc[r * (H / 16) + c / 16] - 127;
      }
#pragma unroll
      for (int u = 0; u < 4; u++) combine_add(s, v[u], ex[u]);
    }
    for (; j < k; j++) {
      const int64_t r = pair_prow[t * k + j];
      const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(o16 + r * H + c));
      combine_add(s, v, (int)osc[r * (H / 16) + c / 16] - 127);
    }
    u32x4_t o;
#pragma unroll
    for (int q = 0; q < 4; q++) o[q] = f32_to_bf16_bits(s[2 * q]) | (f32_to_bf16_bits(s[2 * q + 1]) << 16);
    reinterpret_cast<u32x4_t*>(y)[i] = o;
  }
}

}  // namespace

int launch_gemm1(int af, int NRG, const GemmArgs& a, int64_t max_tiles, hipStream_t stream) {
  return af == kActBf16 ? gemm1_launch<kActBf16>(NRG, a, max_tiles, stream) : launch_gemm1_mx(af, NRG, a, max_tiles, stream);
}

int launch_gemm2(int af, int NRG, const GemmArgs& a, int64_t max_tiles, hipStream_t stream) {
  return af == kActBf16 ? gemm2_launch<kActBf16>(NRG, a, max_tiles, stream) : launch_gemm2_mx(af, NRG, a, max_tiles, stream);
}

int launch_combine(const uint16_t* o16, const uint8_t* osc, const int32_t* pair_prow, void* y, int64_t T, int64_t H, int k,
                   hipStream_t stream) {
  const int64_t n = T * (H / 8);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (n > 0)
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, o16, osc, pair_prow, (uint16_t*)y, H,
                       k, n);
  return hipGetLastError() == hipSuccess ? MXFP4_OK : MXFP4_ERR_DEVICE;
}
