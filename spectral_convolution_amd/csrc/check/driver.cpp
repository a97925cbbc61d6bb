// driver.cpp - the bounds-check build's driver: every public entry point on a
// spread of shapes (matrix-core and VALU planes, 2D and 3D, the three dtypes,
// ragged modes and channels, both launch shapes, the half exchange, the
// backward pass (from x and from saved spectra), weight repacking, the
// allocation-free entry, the FNO block
// and the full FNO2d network). Each launch is checked by its launcher's
// bounds hook against the recording runtime's allocations; the program exits
// non-zero if any span or assumption was broken. Host code only.

#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <vector>

#include "../../../include/fno.h"
#include "../common.hpp"

long check_launches();
long check_reports();

namespace {

int n_fail = 0;

void expect(bool ok, const char *what, int line) {
  if (!ok) {
    std::fprintf(stderr, "driver: line %d: %s\n", line, what);
    ++n_fail;
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)

size_t es_of(fno_dtype_t d) { return d == FNO_F32 ? 4 : 2; }

struct Buf {
  void *p = nullptr;
  explicit Buf(size_t n);
  ~Buf();
};

}  // namespace

Buf::Buf(size_t n) {
  if (hipMalloc(&p, n) != hipSuccess) p = nullptr;
}
Buf::~Buf() { (void)hipFree(p); }

namespace {

void run_layer(int ndim, int B, int Ci, int Co, std::vector<int> grid, std::vector<int> modes, fno_dtype_t dt) {
  fno_plan_t p = nullptr;
  const fno_status_t st = fno_plan_create(&p, ndim, B, Ci, Co, grid.data(), modes.data(), dt, 0);
  if (st == FNO_ERR_UNSUPPORTED) return;
  EXPECT(st == FNO_OK);
  if (st != FNO_OK) return;
  size_t px = 1, K = ndim == 2 ? 2 : 4;
  for (int d = 0; d < ndim; ++d) {
    px *= (size_t)grid[d];
    K *= (size_t)modes[d];
  }
  const size_t es = es_of(dt);
  Buf x((size_t)B * Ci * px * es), y((size_t)B * Co * px * es), w(K * Ci * Co * 2 * es);
  Buf gy((size_t)B * Co * px * es), gx((size_t)B * Ci * px * es), gw(K * Ci * Co * 2 * es);
  auto conv = ndim == 2 ? fno_spectral_conv2d : fno_spectral_conv3d;
  EXPECT(conv(p, x.p, w.p, y.p, nullptr) == FNO_OK);
  auto bwd = ndim == 2 ? fno_spectral_conv2d_backward : fno_spectral_conv3d_backward;
  EXPECT(bwd(p, x.p, w.p, gy.p, gx.p, gw.p, nullptr) == FNO_OK);
  EXPECT(bwd(p, x.p, w.p, gy.p, gx.p, nullptr, nullptr) == FNO_OK);
  EXPECT(bwd(p, x.p, w.p, gy.p, nullptr, gw.p, nullptr) == FNO_OK);
  // the saved-spectra pair, where the plan has a saved format
  size_t sb = 0;
  const fno_status_t ss = fno_plan_saved_bytes(p, &sb);
  EXPECT(ss == FNO_OK || ss == FNO_ERR_UNSUPPORTED);
  if (ss == FNO_OK) {
    Buf sv(sb);
    EXPECT(fno_spectral_conv_forward_save(p, x.p, w.p, y.p, sv.p, nullptr) == FNO_OK);
    EXPECT(fno_spectral_conv_backward_saved(p, sv.p, w.p, gy.p, gx.p, gw.p, nullptr) == FNO_OK);
    EXPECT(fno_spectral_conv_backward_saved(p, sv.p, nullptr, gy.p, nullptr, gw.p, nullptr) == FNO_OK);
  }
  const fno_status_t na = fno_spectral_conv_noalloc(p, x.p, w.p, y.p, nullptr);
  EXPECT(na == FNO_OK || na == FNO_ERR_UNSUPPORTED);
  int nl = 0;
  EXPECT(fno_plan_num_launches(p, &nl) == FNO_OK);
  for (int i = 0; i < nl; ++i) EXPECT(fno_plan_run_launch(p, i, x.p, w.p, y.p, nullptr) == FNO_OK);
  if (fno_plan_set_launch_shape(p, FNO_LAUNCH_FUSED) == FNO_OK) {
    EXPECT(conv(p, x.p, w.p, y.p, nullptr) == FNO_OK);
    if (fno_plan_set_launch_shape(p, FNO_LAUNCH_FUSED_STALL_TEST) == FNO_OK) (void)conv(p, x.p, w.p, y.p, nullptr);
    EXPECT(fno_plan_set_launch_shape(p, FNO_LAUNCH_SEPARATE) == FNO_OK);
  }
  const size_t n = K * Ci * Co;
  Buf re(n * es), im(n * es), corners(2 * n * es);
  EXPECT(fno_weights_pack(p, FNO_WEIGHTS_SPLIT, re.p, im.p, w.p, nullptr) == FNO_OK);
  EXPECT(fno_weights_unpack(p, FNO_WEIGHTS_SPLIT, w.p, re.p, im.p, nullptr) == FNO_OK);
  EXPECT(fno_weights_pack(p, FNO_WEIGHTS_CORNERS, corners.p, nullptr, w.p, nullptr) == FNO_OK);
  EXPECT(fno_weights_unpack(p, FNO_WEIGHTS_CORNERS, w.p, corners.p, nullptr, nullptr) == FNO_OK);
  if (ndim == 2) {
    Buf A((size_t)Co * Ci * es), bias((size_t)Co * es);
    const fno_status_t b0 = fno_block2d(p, x.p, w.p, A.p, bias.p, 1, y.p, nullptr);
    EXPECT(b0 == FNO_OK || b0 == FNO_ERR_UNSUPPORTED);
    if (b0 == FNO_OK) EXPECT(fno_block2d(p, x.p, w.p, A.p, nullptr, 0, y.p, nullptr) == FNO_OK);
  }
  EXPECT(fno_plan_destroy(p) == FNO_OK);
}

void run_model(int B, int H, int W, int in, int ch, int layers, int m1, int m2, int proj, int out, fno_dtype_t dt) {
  fno_model2d_t m = nullptr;
  const fno_status_t st = fno_model2d_create(&m, B, H, W, in, ch, layers, m1, m2, proj, out, dt, 0);
  EXPECT(st == FNO_OK);
  if (st != FNO_OK) return;
  const size_t es = es_of(dt), px = (size_t)H * W, K = (size_t)2 * m1 * m2;
  std::vector<Buf *> bufs;
  auto mk = [&](size_t n) {
    bufs.push_back(new Buf(n * es));
    return bufs.back()->p;
  };
  std::vector<const void *> params;
  params.push_back(mk((size_t)ch * in));
  params.push_back(mk(ch));
  for (int l = 0; l < layers; ++l) {
    params.push_back(mk(K * ch * ch * 2));
    params.push_back(mk((size_t)ch * ch));
    params.push_back(mk(ch));
  }
  params.push_back(mk((size_t)proj * ch));
  params.push_back(mk(proj));
  params.push_back(mk((size_t)out * proj));
  params.push_back(mk(out));
  void *f = mk((size_t)B * in * px), *o = mk((size_t)B * out * px);
  EXPECT(fno_model2d_forward(m, f, params.data(), o, nullptr) == FNO_OK);
  EXPECT(fno_model2d_set_graph(m, 1) == FNO_OK);
  EXPECT(fno_model2d_forward(m, f, params.data(), o, nullptr) == FNO_OK);
  EXPECT(fno_model2d_destroy(m) == FNO_OK);
  for (Buf *b : bufs) delete b;
}

}  // namespace

int main() {
  const fno_dtype_t dts[3] = {FNO_F32, FNO_F16, FNO_BF16};
  // 2D: matrix-core planes (64 .. 256) and the VALU planes (small and
  // non-power-of-two grids), ragged and maximal modes, small and large batches
  struct L2 { int B, Ci, Co, H, W, m1, m2; };
  const L2 l2[] = {
      {2, 4, 4, 16, 16, 4, 4},      {16, 32, 32, 128, 128, 16, 16}, {32, 64, 64, 256, 256, 32, 32},
      {3, 5, 7, 64, 64, 5, 7},      {1, 3, 64, 128, 128, 16, 16},   {20, 64, 64, 256, 256, 24, 24},
      {17, 33, 20, 64, 128, 20, 24}, {2, 8, 12, 32, 48, 6, 9},      {16, 64, 68, 256, 128, 32, 17},
      {1, 1, 1, 64, 64, 1, 1},      {4, 16, 16, 256, 64, 32, 32},   {2, 64, 65, 128, 256, 9, 3},
  };
  for (const L2 &c : l2)
    for (fno_dtype_t dt : dts) run_layer(2, c.B, c.Ci, c.Co, {c.H, c.W}, {c.m1, c.m2}, dt);
  struct L3 { int B, Ci, Co, X, Y, Z, m1, m2, m3; };
  const L3 l3[] = {
      {4, 32, 32, 64, 64, 64, 16, 16, 16}, {2, 3, 5, 16, 16, 16, 4, 4, 4}, {1, 8, 8, 32, 64, 64, 6, 10, 17},
  };
  for (const L3 &c : l3)
    for (fno_dtype_t dt : dts) run_layer(3, c.B, c.Ci, c.Co, {c.X, c.Y, c.Z}, {c.m1, c.m2, c.m3}, dt);
  run_model(2, 64, 64, 3, 32, 2, 8, 8, 16, 1, FNO_F16);
  run_model(20, 256, 256, 3, 64, 4, 24, 24, 128, 1, FNO_F16);
  run_model(1, 64, 64, 3, 64, 4, 12, 12, 128, 1, FNO_BF16);
  run_model(2, 32, 32, 3, 16, 1, 4, 4, 8, 2, FNO_F32);
  run_model(2, 64, 64, 3, 16, 0, 4, 4, 8, 1, FNO_F16);
  const long reports = check_reports();
  // the checker itself: spans past the end of a buffer must be reported
  {
    Buf x(64 * 2), A(4 * 2), y(64 * 2);
    std::fprintf(stderr, "self-test: three planted out-of-range spans follow\n");
    const long before = check_reports();
    fno::check_channel_mix(x.p, A.p, nullptr, nullptr, y.p, 1, 1, 4, 16, fno::DT_F16);  // in range
    EXPECT(check_reports() == before);
    fno::check_channel_mix(x.p, A.p, nullptr, nullptr, y.p, 1, 1, 4, 17, fno::DT_F16);  // y 4 elements short
    EXPECT(check_reports() == before + 1);
    fno::check_channel_mix(x.p, A.p, nullptr, nullptr, y.p, 1, 1, 5, 16, fno::DT_F16);  // A and y a row short
    EXPECT(check_reports() == before + 3);
  }
  std::printf("launches checked: %ld, bounds reports: %ld, driver failures: %d\n", check_launches(), reports,
              n_fail);
  return (reports == 0 && n_fail == 0 && check_launches() > 0) ? 0 : 1;
}
