// The quantized-activation instantiations of the grouped GEMM kernels (gemm_kernel.h): MXFP8 (E4M3)
// and MXFP4 (E2M1) activations, one term per block.  A separate source so the formats compile in
// parallel.
#include "gemm_kernel.h"

int launch_gemm1_mx(int af, int NRG, const GemmArgs& a, int64_t max_tiles, hipStream_t stream) {
  if (af == kActMxfp8) return gemm1_launch<kActMxfp8>(NRG, a, max_tiles, stream);
  if (af == kActMxfp4) return gemm1_launch<kActMxfp4>(NRG, a, max_tiles, stream);
  return MXFP4_ERR_SHAPE;
}

int launch_gemm2_mx(int af, int NRG, const GemmArgs& a, int64_t max_tiles, hipStream_t stream) {
  if (af == kActMxfp8) return gemm2_launch<kActMxfp8>(NRG, a, max_tiles, stream);
  if (af == kActMxfp4) return gemm2_launch<kActMxfp4>(NRG, a, max_tiles, stream);
  return MXFP4_ERR_SHAPE;
}
