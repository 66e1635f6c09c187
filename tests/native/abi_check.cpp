// Calls every entry point of the C ABI with valid and invalid arguments on the CPU (the kernel
// launchers and HIP calls are stand-ins, see abi_stubs.cpp) and checks the returned status, the
// launches made, and that every region carved out of a workspace or blob lies inside it.  Built with
// AddressSanitizer and UndefinedBehaviorSanitizer (-fno-sanitize-recover) by tests/test_abi_sanitized.py.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "abi_stubs.h"

static int g_fail = 0;
#define CHECK(c)                                                    \
  do {                                                              \
    if (!(c)) {                                                     \
      std::printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #c);      \
      g_fail++;                                                     \
    }                                                               \
  } while (0)

// Addresses that are never dereferenced by the validation (the launchers are stand-ins).
static void* fake(uintptr_t off = 0) { return (void*)((uintptr_t(1) << 32) + off); }

static std::vector<std::string> names() {
  std::vector<std::string> v;
  for (auto& c : g_calls) v.push_back(c.name);
  return v;
}

static bool inside(const void* p, size_t bytes_at_p, const void* base, size_t total) {
  const uintptr_t a = (uintptr_t)p, b = (uintptr_t)base;
  return a >= b && a + bytes_at_p <= b + total;
}

static void test_quantize() {
  CHECK(mxfp4_quantize(fake(), 4, 48, 64, fake(), nullptr, nullptr, nullptr) == MXFP4_ERR_SHAPE);
  CHECK(mxfp4_quantize(fake(), 4, 64, 60, fake(), nullptr, nullptr, nullptr) == MXFP4_ERR_SHAPE);
  CHECK(mxfp4_quantize(fake(), -3, 64, 64, fake(), nullptr, nullptr, nullptr) == MXFP4_ERR_SHAPE);
  CHECK(mxfp4_quantize(fake(), INT64_MAX, 64, 64, fake(), nullptr, nullptr, nullptr) == MXFP4_ERR_SHAPE);
  CHECK(mxfp4_quantize(fake(), 4, INT64_MAX - 31, INT64_MAX - 31, fake(), nullptr, nullptr, nullptr) ==
        MXFP4_ERR_SHAPE);
  CHECK(mxfp4_quantize(nullptr, 4, 64, 64, fake(), nullptr, nullptr, nullptr) == MXFP4_ERR_NULL);
  CHECK(mxfp4_quantize(fake(8), 4, 64, 64, fake(), nullptr, nullptr, nullptr) == MXFP4_ERR_ALIGN);
  CHECK(mxfp4_quantize(fake(), 4, 64, 64, fake(), nullptr, fake(4), nullptr) == MXFP4_ERR_ALIGN);
  g_calls.clear();
  CHECK(mxfp4_quantize(nullptr, 0, 64, 64, nullptr, nullptr, nullptr, nullptr) == MXFP4_OK);
  CHECK(g_calls.empty());
  // flat scales at any byte offset are accepted
  CHECK(mxfp4_quantize(fake(), 300, 4128, 4136, fake(), fake(3), fake(16), nullptr) == MXFP4_OK);
  CHECK(g_calls.size() == 1 && g_calls[0].name == "quantize" && g_calls[0].p[2] == fake(3) && g_calls[0].i[0] == 300);
  CHECK(mxfp4_tiled_scale_bytes(8192, 7168) == 64u * 56 * 512);
  CHECK(mxfp4_tiled_scale_bytes(INT64_MAX, 64) == 0 || mxfp4_tiled_scale_bytes(INT64_MAX, 64) > 0);
  CHECK(mxfp4_tiled_scale_bytes(-1, 64) == 0);
}

static void test_nvfp4() {
  CHECK(nvfp4_quantize(fake(), 4, 40, 48, 1.0f, fake(), nullptr, nullptr, nullptr) == MXFP4_ERR_SHAPE);  // K % 16
  CHECK(nvfp4_quantize(fake(), 4, 64, 64, 0.0f, fake(), nullptr, nullptr, nullptr) == MXFP4_ERR_SHAPE);
  CHECK(nvfp4_quantize(fake(), 4, 64, 64, -2.0f, fake(), nullptr, nullptr, nullptr) == MXFP4_ERR_SHAPE);
  CHECK(nvfp4_quantize(fake(), 4, 64, 64, __builtin_nanf(""), fake(), nullptr, nullptr, nullptr) == MXFP4_ERR_SHAPE);
  CHECK(nvfp4_quantize(fake(), 4, 64, 64, __builtin_inff(), fake(), nullptr, nullptr, nullptr) == MXFP4_ERR_SHAPE);
  CHECK(nvfp4_quantize(fake(), INT64_MAX, 64, 64, 1.0f, fake(), nullptr, nullptr, nullptr) == MXFP4_ERR_SHAPE);
  CHECK(nvfp4_quantize(nullptr, 4, 64, 64, 1.0f, fake(), nullptr, nullptr, nullptr) == MXFP4_ERR_NULL);
  CHECK(nvfp4_quantize(fake(8), 4, 64, 64, 1.0f, fake(), nullptr, nullptr, nullptr) == MXFP4_ERR_ALIGN);
  CHECK(nvfp4_quantize(fake(), 4, 64, 64, 1.0f, fake(), nullptr, fake(8), nullptr) == MXFP4_ERR_ALIGN);
  g_calls.clear();
  CHECK(nvfp4_quantize(nullptr, 0, 64, 64, 1.0f, nullptr, nullptr, nullptr, nullptr) == MXFP4_OK);
  CHECK(g_calls.empty());
  CHECK(nvfp4_quantize(fake(), 130, 80, 88, 2.5f, fake(), fake(1), fake(16), nullptr) == MXFP4_OK);
  CHECK(g_calls.size() == 1 && g_calls[0].name == "nvfp4_quantize" && g_calls[0].i[3] == 2560 &&
        g_calls[0].p[2] == fake(1));
  CHECK(nvfp4_tiled_scale_bytes(8192, 7168) == 64u * 112 * 512);
  CHECK(nvfp4_tiled_scale_bytes(129, 80) == 2u * 2 * 512);
  CHECK(nvfp4_tiled_scale_bytes(1, 40) == 0 && nvfp4_tiled_scale_bytes(INT64_MAX, 64) == 0);
}

static void test_linear() {
  CHECK(mxfp4_linear_pack_bytes(2048, 2048, 1) > 0);
  CHECK(mxfp4_linear_pack_bytes(2040, 2048, 0) == 0 && mxfp4_linear_pack_bytes(2048, 16, 0) == 0);
  CHECK(mxfp4_linear_pack_bytes(INT64_MAX, 64, 0) == 0 && mxfp4_linear_pack_bytes(64, 64, 3) == 0);
  const int64_t N = 96, K = 160, M = 70;
  const size_t nb = mxfp4_linear_pack_bytes(N, K, 1);
  CHECK(mxfp4_linear_pack(N, K, fake(), fake(), fake(), 1, fake(), nb - 1, nullptr) == MXFP4_ERR_WORKSPACE);
  CHECK(mxfp4_linear_pack(N, K, fake(8), fake(), nullptr, 0, fake(), nb, nullptr) == MXFP4_ERR_ALIGN);
  CHECK(mxfp4_linear_pack(N, K, nullptr, fake(), nullptr, 0, fake(), nb, nullptr) == MXFP4_ERR_NULL);
  g_calls.clear();
  CHECK(mxfp4_linear_pack(N, K, fake(), fake(), fake(), 1, fake(), nb, nullptr) == MXFP4_OK);
  CHECK(g_calls.size() == 1 && g_calls[0].name == "pack_linear" && (size_t)g_calls[0].i[0] == nb);
  const size_t nw = mxfp4_linear_workspace_bytes(M, N, K);
  CHECK(nw > 0 && mxfp4_linear_workspace_bytes(-1, N, K) == 0);
  void* ws = fake(1ull << 40);
  void* blob = fake(1ull << 36);
  CHECK(mxfp4_linear_forward(blob, N, K, 1, fake(), M, K, fake(), ws, nw - 1, nullptr) == MXFP4_ERR_WORKSPACE);
  CHECK(mxfp4_linear_forward(blob, N, K, 1, fake(), M, K - 8, fake(), ws, nw, nullptr) == MXFP4_ERR_SHAPE);
  CHECK(mxfp4_linear_forward(blob, N, K, 1, fake(2), M, K, fake(), ws, nw, nullptr) == MXFP4_ERR_ALIGN);
  CHECK(mxfp4_linear_forward(blob, N, K, 2, fake(), M, K, fake(), ws, nw, nullptr) == MXFP4_ERR_SHAPE);
  g_calls.clear();
  CHECK(mxfp4_linear_forward(nullptr, N, K, 1, nullptr, 0, K, nullptr, nullptr, 0, nullptr) == MXFP4_OK);
  CHECK(g_calls.empty());
  CHECK(mxfp4_linear_forward(blob, N, K, 1, fake(), M, K, fake(), ws, nw, nullptr) == MXFP4_OK);
  CHECK((names() == std::vector<std::string>{"linear_prep", "gemm2"}));
  if (g_calls.size() == 2) {
    const GemmArgs& a = g_calls[1].gemm;
    const MoeGeom g = moe_geom(1, N, K);
    const LinearOffsets o = linear_offsets(g, true);
    const LinearWs w = linear_ws(M, g);
    CHECK(a.ydense == fake() && a.o16 == nullptr && g_calls[1].i[0] == 1 && g_calls[1].i[1] == w.nrg);
    CHECK(inside(a.wq, (size_t)g.ncb2 * g.nkt2 * kCB * 1024, blob, o.total));
    CHECK(inside(a.ws, (size_t)g.ncb2 * g.nkt2 * 1024, blob, o.total));
    CHECK(inside(a.bias, (size_t)N * 2, blob, o.total));
    CHECK(inside(a.xq, (size_t)w.nrg * g.nkt2 * 64 * kMaxSlot, ws, nw));
    CHECK(inside(a.xs, (size_t)w.nrg * g.nkt2 * 64 * 4, ws, nw));
    CHECK(inside(a.prow_w, 4 * ((size_t)w.nrg * 32 + 64), ws, nw));
    CHECK(inside(a.tiles, 16 * (size_t)w.nrg, ws, nw) && inside(a.ntiles, 4, ws, nw));
    CHECK(a.ntl == N / 32 && a.H == N && a.nkt == (K + 63) / 64);
  }
  // the split activations must stay addressable with 32-bit offsets
  CHECK(mxfp4_linear_forward(blob, 64, 1 << 20, 0, fake(), 4096, 1 << 20, fake(), ws, SIZE_MAX, nullptr) ==
        MXFP4_ERR_SHAPE);
}

static void test_repack() {
  mxfp4_moe_dims d = {4, 256, 128, 1};
  CHECK(mxfp4_repack_bytes(&d, 0) > 0);
  CHECK(mxfp4_repack_bytes(&d, 4) == 0);
  CHECK(mxfp4_repack_bytes(nullptr, 0) == 0);
  mxfp4_moe_dims big = {1 << 30, 1 << 30, 1 << 30, 0};
  CHECK(mxfp4_repack_bytes(&big, 0) == 0);
  mxfp4_moe_dims neg = {-4, 256, 128, 0};
  CHECK(mxfp4_repack_bytes(&neg, 0) == 0);
  // checked-conversion offsets: the page's order w13, w2, w13 scale, w2 scale, b13, b2
  size_t off[6];
  CHECK(mxfp4_repack_offsets(&d, MXFP4_LAYOUT_STD_W31, off) == MXFP4_OK);
  const size_t E = 4, H = 256, I = 128;
  CHECK(off[0] == 0);
  CHECK(off[1] >= off[0] + E * 2 * I * H / 2);
  CHECK(off[2] >= off[1] + E * H * I / 2);
  CHECK(off[3] >= off[2] + E * 2 * I * H / 32);
  CHECK(off[4] >= off[3] + E * H * I / 32);
  CHECK(off[5] >= off[4] + E * 2 * I * 2);
  CHECK(mxfp4_repack_bytes(&d, MXFP4_LAYOUT_STD_W31) >= off[5] + E * H * 2);
  for (int k = 0; k < 6; k++) CHECK(off[k] % 256 == 0);
  CHECK(mxfp4_repack_offsets(&d, MXFP4_LAYOUT_GFX950, off) == MXFP4_ERR_LAYOUT);
  CHECK(mxfp4_repack_offsets(&d, MXFP4_LAYOUT_STD_W31, nullptr) == MXFP4_ERR_NULL);
  const size_t n = mxfp4_repack_bytes(&d, 0);
  CHECK(mxfp4_repack_weights(&d, fake(), fake(), fake(), fake(), nullptr, nullptr, 1, 0, fake(), n, nullptr) ==
        MXFP4_ERR_NULL);  // biases missing
  CHECK(mxfp4_repack_weights(&d, fake(), fake(), fake(), fake(), fake(2), fake(), 1, 0, fake(), n, nullptr) ==
        MXFP4_ERR_ALIGN);  // fp32 bias at 2 bytes
  CHECK(mxfp4_repack_weights(&d, fake(), fake(), fake(), fake(), fake(), fake(), 1, 0, fake(), n - 1, nullptr) ==
        MXFP4_ERR_WORKSPACE);
  CHECK(mxfp4_repack_weights(&d, fake(), fake(), fake(), fake(), fake(), fake(), 1, 3 | 4, fake(), n, nullptr) ==
        MXFP4_ERR_LAYOUT);
  g_calls.clear();
  CHECK(mxfp4_repack_weights(&d, fake(), fake(), fake(), fake(), fake(), fake(), 1, 0, fake(), n, nullptr) == MXFP4_OK);
  CHECK(g_calls.size() == 1 && g_calls[0].name == "repack_gfx950" && (size_t)g_calls[0].i[0] == n);
  const uint32_t lay = MXFP4_LAYOUT_STD_W31 | MXFP4_LAYOUT_SCALE_TILED;
  const size_t ns = mxfp4_repack_bytes(&d, lay);
  g_calls.clear();
  CHECK(mxfp4_repack_weights(&d, fake(), fake(), fake(), fake(), fake(), fake(), 0, lay, fake(), ns, nullptr) ==
        MXFP4_OK);
  CHECK(g_calls.size() == 1 && g_calls[0].name == "repack_standard" && g_calls[0].i[0] == 1 && g_calls[0].i[1] == 1);
  for (int k = 0; k < 6; k++) CHECK(g_calls[0].off[k] < ns);
}

static void test_header_checks() {
  mxfp4_moe_dims d = {3, 96, 96, 1};
  const MoeGeom g = moe_geom(d.E, d.H, d.I);
  const BlobOffsets o = blob_offsets(g, true);
  // a blob header as the repack writes it, in host memory standing in for the device
  std::vector<uint8_t> raw(512 + 256);
  uint8_t* blob = raw.data() + (256 - ((uintptr_t)raw.data() & 255));
  BlobHeader h;
  std::memset(&h, 0, sizeof h);
  std::memcpy(h.magic, MX_BLOB_MAGIC, 8);
  h.version = MX_BLOB_VERSION;
  h.E = d.E; h.H = d.H; h.I = d.I; h.has_bias = d.has_bias;
  h.off_w13q = o.w13q; h.off_w13s = o.w13s; h.off_w2q = o.w2q; h.off_w2s = o.w2s;
  h.off_b13 = o.b13; h.off_b2 = o.b2; h.total = o.total;
  std::memcpy(blob, &h, sizeof h);
  CHECK(mxfp4_check_packed(&d, blob, nullptr) == MXFP4_OK);
  mxfp4_moe_dims d2 = d;
  d2.I = 128;
  CHECK(mxfp4_check_packed(&d2, blob, nullptr) == MXFP4_ERR_LAYOUT);
  d2 = d;
  d2.has_bias = 0;
  CHECK(mxfp4_check_packed(&d2, blob, nullptr) == MXFP4_ERR_LAYOUT);
  CHECK(mxfp4_check_packed(&d, blob + 16, nullptr) == MXFP4_ERR_ALIGN);
  CHECK(mxfp4_check_packed(&d, nullptr, nullptr) == MXFP4_ERR_NULL);
  g_calls.clear();
  CHECK(mxfp4_unpack_weights(&d, blob, fake(), fake(), fake(), fake(), fake(), fake(), nullptr) == MXFP4_OK);
  CHECK(g_calls.size() == 1 && g_calls[0].name == "unpack_gfx950" && g_calls[0].p[0] == blob);
  blob[0] ^= 1;  // a corrupted magic
  CHECK(mxfp4_check_packed(&d, blob, nullptr) == MXFP4_ERR_LAYOUT);
  g_calls.clear();
  CHECK(mxfp4_unpack_weights(&d, blob, fake(), fake(), fake(), fake(), fake(), fake(), nullptr) == MXFP4_ERR_LAYOUT);
  CHECK(g_calls.empty());
}

static void test_route() {
  CHECK(moe_mxfp4_route_workspace_bytes(64, 128, 8) > 0);
  CHECK(moe_mxfp4_route_workspace_bytes(64, 128, 33) == 0);
  CHECK(moe_mxfp4_route_workspace_bytes(-1, 128, 8) == 0);
  CHECK(moe_mxfp4_route_workspace_bytes(INT64_MAX / 2, 128, 8) == 0);
  const int64_t T = 1000;
  const int E = 300, k = 7;
  const size_t n = moe_mxfp4_route_workspace_bytes(T, E, k);
  std::vector<uint8_t> raw(n + 256);
  void* ws = raw.data() + (256 - ((uintptr_t)raw.data() & 255));
  float* lg = (float*)fake();
  int32_t* ids = (int32_t*)fake(1 << 24);
  float* w = (float*)fake(2 << 24);
  int32_t* offs = (int32_t*)fake(3 << 24);
  int32_t* sp = (int32_t*)fake(4 << 24);
  CHECK(moe_mxfp4_route(lg, T, E, k, 1, ids, w, offs, sp, ws, n - 1, nullptr) == MXFP4_ERR_WORKSPACE);
  CHECK(moe_mxfp4_route(lg, T, E, k, 1, ids, w, offs, sp, (uint8_t*)ws + 4, n, nullptr) == MXFP4_ERR_ALIGN);
  CHECK(moe_mxfp4_route(lg, T, E, k, 1, ids, w, offs, nullptr, ws, n, nullptr) == MXFP4_ERR_NULL);
  g_calls.clear();
  CHECK(moe_mxfp4_route(lg, T, E, k, 1, ids, w, offs, sp, ws, n, nullptr) == MXFP4_OK);
  CHECK((names() == std::vector<std::string>{"route", "place"}));
  // every table the launches use lies inside the workspace; the routing writes the histograms the
  // placement reads
  const Call& rt = g_calls[0];
  const Call& pl = g_calls[1];
  CHECK(rt.p[3] == pl.p[0] && rt.p[4] == pl.p[12] && rt.i[0] == T && rt.i[1] == E && rt.i[2] == k);
  CHECK(inside(rt.p[4], 4 * T * k, ws, n));
  const int64_t nrows = ((T * k + 31 * E + 31) / 32) * 32 + 128;
  CHECK(inside(pl.p[0], 4 * cdiv(T, kRouteTokens) * E, ws, n));
  CHECK(inside(pl.p[2], 4 * (E + 1), ws, n));
  for (int q = 4; q <= 6; q++) CHECK(inside(pl.p[q], 4 * nrows, ws, n));
  CHECK(inside(pl.p[8], 16 * (cdiv(T * k, 32) + E), ws, n));
  CHECK(inside(pl.p[9], 4, ws, n));
}

static void check_forward_layout(const mxfp4_moe_dims& d, int64_t T, int k, size_t nws, const void* ws,
                                 const void* blob) {
  const MoeGeom g = moe_geom(d.E, d.H, d.I);
  const FwdWs w = fwd_ws(g, T, k);
  const BlobOffsets o = blob_offsets(g, d.has_bias);
  CHECK(w.total <= nws);
  CHECK((names() == std::vector<std::string>{"front", "place", "gemm1", "gemm2", "combine"}));
  if (g_calls.size() != 5) return;
  const Call& fr = g_calls[0];
  CHECK(inside(fr.p[1], (size_t)T * g.nkt1 * kMaxRec, ws, nws));
  CHECK(inside(fr.p[2], 4 * (size_t)((T + kRouteTokens - 1) / kRouteTokens) * fr.i[2], ws, nws));
  CHECK(fr.i[2] == d.E && fr.i[4] == k && fr.p[2] == g_calls[1].p[0] && fr.p[6] == g_calls[1].p[12]);
  CHECK(fr.p[6] == g_calls[1].p[7]);  // the ranks live in pair_prow until the placement overwrites them
  CHECK(inside(fr.p[4], 4 * (size_t)T * k, ws, nws) && inside(fr.p[5], 4 * (size_t)T * k, ws, nws));
  const GemmArgs& a1 = g_calls[2].gemm;
  const GemmArgs& a2 = g_calls[3].gemm;
  CHECK(inside(a1.wq, (size_t)g.E * g.ncb1 * g.nkt1 * kCB * 1024, blob, o.total));
  CHECK(inside(a1.ws, (size_t)g.E * g.ncb1 * g.nkt1 * 1024, blob, o.total));
  CHECK(inside(a2.wq, (size_t)g.E * g.ncb2 * g.nkt2 * kCB * 1024, blob, o.total));
  CHECK(inside(a2.ws, (size_t)g.E * g.ncb2 * g.nkt2 * 1024, blob, o.total));
  CHECK((a1.bias != nullptr) == (d.has_bias != 0) && (a2.bias != nullptr) == (d.has_bias != 0));
  if (d.has_bias) {
    CHECK(inside(a1.bias, (size_t)g.E * 2 * g.I * 2, blob, o.total));
    CHECK(inside(a2.bias, (size_t)g.E * g.H * 2, blob, o.total));
  }
  CHECK(inside(a1.xq, (size_t)T * g.nkt1 * kMaxRec, ws, nws));
  CHECK(inside(a1.actq, (size_t)(w.nrows_alloc / 32) * g.nkt2 * 64 * kMaxSlot, ws, nws));
  CHECK(inside(a1.acts, (size_t)(w.nrows_alloc / 32) * g.nkt2 * 64 * 4, ws, nws));
  CHECK(a2.xq == a1.actq && a2.xs == a1.acts);
  for (const GemmArgs* a : {&a1, &a2}) {
    CHECK(inside(a->prow_tok, 4 * w.nrows_alloc, ws, nws));
    CHECK(inside(a->prow_pair, 4 * w.nrows_alloc, ws, nws));
    CHECK(inside(a->prow_w, 4 * w.nrows_alloc, ws, nws));
    CHECK(inside(a->tiles, 16 * w.max_tiles, ws, nws));
    CHECK(inside(a->ntiles, 4, ws, nws));
  }
  CHECK(inside(a2.o16, (size_t)w.nrows_alloc * g.H * 2, ws, nws));
  CHECK(inside(a2.osc, (size_t)w.nrows_alloc * (g.H / 16), ws, nws));
  CHECK(a1.nkt == g.nkt1 && a2.nkt == g.nkt2 && a1.ncb == g.ncb1 && a2.ncb == g.ncb2);
  const Call& cb = g_calls[4];
  CHECK(cb.p[0] == a2.o16 && cb.p[1] == a2.osc && cb.i[0] == T && cb.i[2] == k);
  CHECK(inside(cb.p[2], 4 * T * k, ws, nws));
}

static void test_forward() {
  struct Case { mxfp4_moe_dims d; int64_t T; int k; };
  const Case cases[] = {{{128, 2048, 768, 1}, 64, 8}, {{128, 2048, 768, 0}, 8192, 8},
                        {{384, 7168, 2048, 0}, 4096, 8}, {{4, 256, 128, 1}, 16, 2}, {{1, 32, 32, 0}, 1, 1},
                        {{1024, 64, 64, 1}, 100, 32}};
  for (const Case& c : cases) {
    const size_t nws = moe_mxfp4_workspace_bytes(&c.d, c.T, c.k);
    CHECK(nws > 0);
    const size_t nblob = mxfp4_repack_bytes(&c.d, 0);
    void* ws = fake(1ull << 40);
    void* blob = fake(1ull << 36);
    void* x = fake(1ull << 30);
    float* lg = (float*)fake(3ull << 30);
    void* y = fake(5ull << 30);
    g_calls.clear();
    CHECK(moe_mxfp4_forward(&c.d, blob, x, c.T, c.d.H, lg, c.k, 1, y, nullptr, nullptr, ws, nws, nullptr) == MXFP4_OK);
    check_forward_layout(c.d, c.T, c.k, nws, ws, blob);
    (void)nblob;
    // argument errors: nothing launched
    g_calls.clear();
    CHECK(moe_mxfp4_forward(&c.d, blob, x, c.T, c.d.H, lg, c.k, 1, y, nullptr, nullptr, ws, nws - 1, nullptr) ==
          MXFP4_ERR_WORKSPACE);
    CHECK(moe_mxfp4_forward(&c.d, blob, x, c.T, c.d.H - 8, lg, c.k, 1, y, nullptr, nullptr, ws, nws, nullptr) ==
          MXFP4_ERR_SHAPE);
    CHECK(moe_mxfp4_forward(&c.d, (uint8_t*)blob + 16, x, c.T, c.d.H, lg, c.k, 1, y, nullptr, nullptr, ws, nws,
                            nullptr) == MXFP4_ERR_ALIGN);
    CHECK(moe_mxfp4_forward(&c.d, blob, x, c.T, c.d.H, lg, c.k + 33, 1, y, nullptr, nullptr, ws, nws, nullptr) ==
          MXFP4_ERR_SHAPE);
    CHECK(g_calls.empty());
    // profiled: one event per stage boundary (6), fewer when fewer are given
    g_events = 0;
    void* evs[6] = {fake(), fake(), fake(), fake(), fake(), fake()};
    CHECK(moe_mxfp4_forward_profiled(&c.d, 0, blob, x, c.T, c.d.H, lg, c.k, 1, y, nullptr, nullptr, ws, nws, nullptr,
                                     evs, 6) == MXFP4_OK);
    CHECK(g_events == 6);
    g_events = 0;
    CHECK(moe_mxfp4_forward_profiled(&c.d, 0, blob, x, c.T, c.d.H, lg, c.k, 1, y, nullptr, nullptr, ws, nws, nullptr,
                                     evs, 3) == MXFP4_OK);
    CHECK(g_events == 3);
    CHECK(moe_mxfp4_forward_profiled(&c.d, 0, blob, x, c.T, c.d.H, lg, c.k, 1, y, nullptr, nullptr, ws, nws, nullptr,
                                     nullptr, 3) == MXFP4_ERR_NULL);
    // every activation format: the same launches on the same workspace, the format passed to the
    // producers and the GEMMs; an unknown format is rejected before any launch
    for (int af = 0; af < 3; af++) {
      g_calls.clear();
      CHECK(moe_mxfp4_forward_act(&c.d, af, blob, x, c.T, c.d.H, lg, c.k, 1, y, nullptr, nullptr, ws, nws, nullptr) ==
            MXFP4_OK);
      check_forward_layout(c.d, c.T, c.k, nws, ws, blob);
      if (g_calls.size() == 5) CHECK(g_calls[0].i[3] == af && g_calls[2].i[2] == af && g_calls[3].i[2] == af);
    }
    g_calls.clear();
    CHECK(moe_mxfp4_forward_act(&c.d, 3, blob, x, c.T, c.d.H, lg, c.k, 1, y, nullptr, nullptr, ws, nws, nullptr) ==
          MXFP4_ERR_LAYOUT);
    CHECK(moe_mxfp4_forward_act(&c.d, -1, blob, x, c.T, c.d.H, lg, c.k, 1, y, nullptr, nullptr, ws, nws, nullptr) ==
          MXFP4_ERR_LAYOUT);
    CHECK(g_calls.empty());
  }
  // no tokens: nothing to do
  mxfp4_moe_dims d = {8, 256, 128, 0};
  g_calls.clear();
  CHECK(moe_mxfp4_forward(&d, nullptr, nullptr, 0, 256, nullptr, 2, 1, nullptr, nullptr, nullptr, nullptr, 0,
                          nullptr) == MXFP4_OK);
  CHECK(g_calls.empty());
  // 32-bit copy offsets: T * H / 64 * 144 bytes of first-GEMM records must stay below 4 GiB
  mxfp4_moe_dims dl = {8, 7168, 2048, 0};
  const int64_t limit = (int64_t(1) << 32) / (7168 / 64 * 144);
  CHECK(moe_mxfp4_forward(&dl, fake(), fake(), limit + 1, 7168, (float*)fake(), 1, 1, fake(), nullptr, nullptr,
                          fake(), SIZE_MAX, nullptr) == MXFP4_ERR_SHAPE);
  CHECK(moe_mxfp4_workspace_bytes(&dl, INT64_MAX / 4, 8) == 0);
}

int main() {
  test_quantize();
  test_nvfp4();
  test_linear();
  test_repack();
  test_header_checks();
  test_route();
  test_forward();
  if (g_fail) {
    std::printf("%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("abi checks passed\n");
  return 0;
}
