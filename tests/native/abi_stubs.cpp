// Stand-ins for the library's kernel launchers and for the HIP runtime calls the argument validation
// makes, so that the validation and workspace-carving code (csrc/api.cpp) builds for the CPU alone
// and runs under AddressSanitizer and UndefinedBehaviorSanitizer.  "Device" pointers are host memory
// here: the header read of a packed blob is a plain memcpy.  Each launcher records its call.
#include <hip/hip_runtime_api.h>

#include <cstring>

#include "abi_stubs.h"

std::vector<Call> g_calls;
int g_events = 0;

static int rec(const char* name, Call c = Call()) {
  c.name = name;
  g_calls.push_back(c);
  return MXFP4_OK;
}

int launch_quantize(const void* x, int64_t M, int64_t K, int64_t ldx, void* q, void* sflat, void* stiled, hipStream_t) {
  Call c;
  c.p[0] = x; c.p[1] = q; c.p[2] = sflat; c.p[3] = stiled;
  c.i[0] = M; c.i[1] = K; c.i[2] = ldx;
  return rec("quantize", c);
}
int launch_nvfp4_quantize(const void* x, int64_t M, int64_t K, int64_t ldx, float gs, void* q, void* sflat,
                          void* stiled, hipStream_t) {
  Call c;
  c.p[0] = x; c.p[1] = q; c.p[2] = sflat; c.p[3] = stiled;
  c.i[0] = M; c.i[1] = K; c.i[2] = ldx; c.i[3] = (int64_t)(gs * 1024.0f);
  return rec("nvfp4_quantize", c);
}
int launch_repack_gfx950(const MoeGeom& g, const BlobOffsets& o, bool bias, const void*, const void*, const void*,
                         const void*, const void*, const void*, int, void* out, hipStream_t) {
  Call c;
  c.p[0] = out; c.i[0] = (int64_t)o.total; c.i[1] = bias; c.i[2] = g.E;
  return rec("repack_gfx950", c);
}
int launch_unpack_gfx950(const MoeGeom& g, const BlobOffsets&, bool bias, const void* packed, void*, void*, void*,
                         void*, void*, void*, hipStream_t) {
  Call c;
  c.p[0] = packed; c.i[0] = g.E; c.i[1] = bias;
  return rec("unpack_gfx950", c);
}
int launch_repack_standard(const MoeGeom& g, bool bias, const void*, const void*, const void*, const void*,
                           const void*, const void*, int, bool swap, bool tiled, const size_t off[6], void* out,
                           hipStream_t) {
  Call c;
  c.p[0] = out; c.i[0] = swap; c.i[1] = tiled; c.i[2] = bias; c.i[3] = g.E;
  for (int k = 0; k < 6; k++) c.off[k] = off[k];
  return rec("repack_standard", c);
}
int launch_pack_linear(const MoeGeom& g, const LinearOffsets& o, bool bias, const void*, const void*, const void*, int,
                       void* out, hipStream_t) {
  Call c;
  c.p[0] = out; c.i[0] = (int64_t)o.total; c.i[1] = bias; c.i[2] = g.H; c.i[3] = g.I;
  return rec("pack_linear", c);
}
int launch_linear_prep(const void* x, int64_t M, int64_t ldx, const MoeGeom&, const LinearWs& w, uint8_t* ws,
                       hipStream_t) {
  Call c;
  c.p[0] = x; c.p[1] = ws; c.i[0] = M; c.i[1] = ldx; c.i[2] = (int64_t)w.total;
  return rec("linear_prep", c);
}
int launch_front(int af, const void* x, int64_t T, int64_t ldx, const MoeGeom&, void* xq, const float* logits, int E,
                 int k, int, int32_t* ids, float* w, int32_t* blkcnt, int32_t* rank, hipStream_t) {
  Call c;
  c.p[0] = x; c.p[1] = xq; c.p[2] = blkcnt; c.p[3] = logits; c.p[4] = ids; c.p[5] = w; c.p[6] = rank;
  c.i[0] = T; c.i[1] = ldx; c.i[2] = E; c.i[3] = af; c.i[4] = k;
  return rec("front", c);
}
int launch_route(const float* logits, int64_t T, int E, int k, int, int32_t* ids, float* w, int32_t* blkcnt,
                 int32_t* rank, hipStream_t) {
  Call c;
  c.p[0] = logits; c.p[1] = ids; c.p[2] = w; c.p[3] = blkcnt; c.p[4] = rank; c.i[0] = T; c.i[1] = E; c.i[2] = k;
  return rec("route", c);
}
int launch_place(const int32_t*, const float*, int32_t* blkcnt, const int32_t* rank, int64_t T, int k, int E, int BM,
                 int BM2, int32_t* offsets, int32_t* poffsets, int32_t* sorted_pairs, int32_t* prow_pair,
                 int32_t* prow_tok, float* prow_w, int32_t* pair_prow, void* tiles, int32_t* ntiles, void* tiles2,
                 int32_t* ntiles2, hipStream_t) {
  Call c;
  c.p[0] = blkcnt; c.p[1] = offsets; c.p[2] = poffsets; c.p[3] = sorted_pairs; c.p[4] = prow_pair;
  c.p[5] = prow_tok; c.p[6] = prow_w; c.p[7] = pair_prow; c.p[8] = tiles; c.p[9] = ntiles; c.p[10] = tiles2;
  c.p[11] = ntiles2; c.p[12] = rank;
  c.i[0] = T; c.i[1] = k; c.i[2] = E; c.i[3] = BM; c.i[4] = BM2;
  return rec("place", c);
}
int launch_gemm1(int af, int NRG, const GemmArgs& a, int64_t max_tiles, hipStream_t) {
  Call c;
  c.gemm = a; c.i[0] = NRG; c.i[1] = max_tiles; c.i[2] = af;
  return rec("gemm1", c);
}
int launch_gemm2(int af, int NRG, const GemmArgs& a, int64_t max_tiles, hipStream_t) {
  Call c;
  c.gemm = a; c.i[0] = NRG; c.i[1] = max_tiles; c.i[2] = af;
  return rec("gemm2", c);
}
int launch_combine(const uint16_t* o16, const uint8_t* osc, const int32_t* pair_prow, void* y, int64_t T, int64_t H, int k,
                   hipStream_t) {
  Call c;
  c.p[0] = o16; c.p[1] = osc; c.p[2] = pair_prow; c.p[3] = y; c.i[0] = T; c.i[1] = H; c.i[2] = k;
  return rec("combine", c);
}

extern "C" {
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind, hipStream_t) {
  std::memcpy(dst, src, n);
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipEventRecord(hipEvent_t, hipStream_t) {
  g_events++;
  return hipSuccess;
}
}
