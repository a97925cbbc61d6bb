// fno_api.cpp - the C ABI: plan validation, tables, workspace and launches.
//
// A 2D layer is three stream-ordered launches:
//   fno_fwd_plane  (pruned r2c along W + pruned c2c along H, scaled)
//   fno_contract   (per-mode complex contraction on MFMA)
//   fno_inv_plane  (pruned c2c along H + pruned c2r along W)
// A 3D layer applies the plane transforms to every x-slab (axes Y, Z) and
// adds the outermost axis as a separate pruned c2c pass:
//   fno_fwd_plane(slabs) -> fno_fwd_axis(X) -> fno_contract ->
//   fno_inv_axis(X) -> fno_inv_plane(slabs)
// Spectra between launches live in the plan's workspace (complex fp32).
//
// The backward pass (gradients of x and w from g = dL/dy) reuses the same
// kernels: dx is the layer applied to g with every mode's weight replaced by
// its conjugate transpose (forward planes of g, the contraction from Co to Ci
// channels reading W transposed, or W^H from fno_conj_transpose where it
// cannot, inverse planes); dw is a per-mode
// reduction over the batch of conj(forward(x)) * forward(g) (fno_grad_w).

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <algorithm>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>
#include <new>
#include <vector>

#include "../../include/fno.h"
#include "common.hpp"

using namespace fno;

namespace fno {

hipError_t raise_lds_cap(const void *k, size_t lds) {
  static std::mutex mu;
  static std::map<std::pair<int, const void *>, size_t> caps;  // (device, kernel) -> allowance
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  size_t &cap = caps[{dev, k}];
  if (lds <= cap) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e == hipSuccess) cap = lds;
  return e;
}

}  // namespace fno

namespace {

constexpr int kMaxAxis = 256;
constexpr int kMinAxis = 8;
constexpr int kMaxRegFFT = 32;
constexpr size_t kMaxLds = 160 * 1024;

enum LaunchKind { L_FWD_PLANE, L_FWD_AXIS, L_CONTRACT, L_INV_AXIS, L_INV_PLANE, L_FUSED };

// Grid-barrier waits of the single-launch layer: polls before giving up
// (each poll sleeps ~128 clocks and reads the barrier word from memory, so
// this is of the order of a second), and the tiny bound of the stall test.
constexpr unsigned kBarrierSpin = 1u << 20;
constexpr unsigned kStallTestSpin = 256;


bool is_pow2(long v) { return v > 0 && (v & (v - 1)) == 0; }
int next_pow2(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

// exp(-2 pi i k / n) for k < n from the definition in double precision: the
// angle is reduced in integers to a quarter turn plus an angle in [0, pi/2),
// whose cos / sin are taken and rotated back by the quarter turns
std::vector<float2> twiddles(int n) {
  std::vector<float2> t(n);
  for (int k = 0; k < n; ++k) {
    const long q = (4L * k) / n;            // quarter turns
    const long rem = 4L * k - q * n;        // remaining angle = (pi/2) * rem / n
    const double a = (M_PI / 2.0) * (double)rem / (double)n;
    const double ca = std::cos(a), sa = std::sin(a);
    double c, s;
    switch (q) {
      case 0: c = ca; s = sa; break;
      case 1: c = -sa; s = ca; break;
      case 2: c = -ca; s = -sa; break;
      default: c = sa; s = -ca; break;
    }
    t[k] = make_float2((float)c, (float)(-s));
  }
  return t;
}

uint16_t half_bits(double v) { return __builtin_bit_cast(uint16_t, (_Float16)v); }

// fp16 parts of table values: hi = fp16(v) and, when lo is given,
// lo = fp16(v - hi) (fp32 plans carry both)
void half_parts(const std::vector<double> &v, std::vector<uint16_t> &hi, std::vector<uint16_t> *lo) {
  hi.resize(v.size());
  if (lo) lo->resize(v.size());
  for (size_t i = 0; i < v.size(); ++i) {
    const _Float16 h = (_Float16)v[i];
    hi[i] = __builtin_bit_cast(uint16_t, h);
    if (lo) (*lo)[i] = half_bits(v[i] - (double)h);
  }
}

// cos and sin of 2 pi k / n (k reduced mod n in integers, quarter turns exact)
void cos_sin_2pi(long k, long n, double &c, double &s) {
  const long r = ((k % n) + n) % n;
  const long q = (4 * r) / n, rem = 4 * r - q * n;
  const double a = (M_PI / 2.0) * (double)rem / (double)n;
  const double ca = std::cos(a), sa = std::sin(a);
  switch (q) {
    case 0: c = ca; s = sa; break;
    case 1: c = -sa; s = ca; break;
    case 2: c = -ca; s = -sa; break;
    default: c = sa; s = -ca; break;
  }
}

// Forward row-DFT fragments, [nt][kb][lane][8] fp16: lane l of tile nt,
// block kb holds T[w][c] for c = 16 nt + l % 16 and w = 32 kb + 8 (l / 16) + i,
// T[w][2 ky] = cos(2 pi ky w / W), T[w][2 ky + 1] = -sin(..), zero for
// ky >= m2 (the A operand of the transposed row product R^T = T^T x^T).
void fwd_fragments(int W, int m2, int NT, std::vector<double> &hi) {
  const int KB = W / 32;
  hi.assign((size_t)NT * KB * 64 * 8, 0);
  for (int nt = 0; nt < NT; ++nt)
    for (int kb = 0; kb < KB; ++kb)
      for (int l = 0; l < 64; ++l)
        for (int i = 0; i < 8; ++i) {
          const int w = kb * 32 + 8 * (l / 16) + i, c = nt * 16 + l % 16, ky = c / 2;
          double v = 0.0;
          if (ky < m2) {
            double cs, sn;
            cos_sin_2pi((long)ky * w, W, cs, sn);
            v = (c & 1) ? -sn : cs;
          }
          hi[(((size_t)nt * KB + kb) * 64 + l) * 8 + i] = v;
        }
}

// Inverse row fragments (B operand, K = c, N = w): [wt][kb][lane][8],
// value T'[c][w] = g cos / -g sin (2 pi ky w / W), g = 1 for ky = 0, else 2.
void inv_fragments(int W, int m2, int KBT, std::vector<double> &tb) {
  const int NWT = W / 16;
  tb.assign((size_t)NWT * KBT * 64 * 8, 0);
  for (int wt = 0; wt < NWT; ++wt)
    for (int kb = 0; kb < KBT; ++kb)
      for (int l = 0; l < 64; ++l)
        for (int i = 0; i < 8; ++i) {
          const int w = wt * 16 + l % 16, c = kb * 32 + 8 * (l / 16) + i, ky = c / 2;
          double v = 0.0;
          if (ky < m2) {
            double cs, sn;
            cos_sin_2pi((long)ky * w, W, cs, sn);
            const double g = ky == 0 ? 1.0 : 2.0;
            v = (c & 1) ? -g * sn : g * cs;
          }
          tb[(((size_t)wt * KBT + kb) * 64 + l) * 8 + i] = v;
        }
}

// Column DFT of one 64-row block, forward (A operand, M = (q, re/im),
// K = (j, re/im)): [mt][kb][lane][8]. Row m = 2q + po, column k = 2j + pi of
// the real form of e^{-i theta}, theta = 2 pi kx(q) j / H:
// [[cos, sin], [-sin, cos]]; zero rows for q >= 2 m1.
void fwd_col_fragments(int H, int m1, int MT, std::vector<double> &ef) {
  ef.assign((size_t)MT * 4 * 64 * 8, 0);
  for (int mt = 0; mt < MT; ++mt)
    for (int kb = 0; kb < 4; ++kb)
      for (int l = 0; l < 64; ++l)
        for (int i = 0; i < 8; ++i) {
          const int m = mt * 16 + l % 16, k = kb * 32 + 8 * (l / 16) + i;
          const int q = m >> 1, po = m & 1, j = k >> 1, pi = k & 1;
          double v = 0.0;
          if (q < 2 * m1) {
            const int kx = q < m1 ? q : H - 2 * m1 + q;
            double cs, sn;
            cos_sin_2pi((long)kx * j, H, cs, sn);
            v = po == 0 ? (pi == 0 ? cs : sn) : (pi == 0 ? -sn : cs);
          }
          ef[(((size_t)mt * 4 + kb) * 64 + l) * 8 + i] = v;
        }
}

// Column DFT of one 64-row block, inverse (A operand, M = (j, re/im),
// K = (q, re/im)): [8][kb1][lane][8], real form of e^{+i theta}:
// [[cos, -sin], [sin, cos]]; zero columns for q >= 2 m1.
void inv_col_fragments(int H, int m1, int KB1, std::vector<double> &ef) {
  ef.assign((size_t)8 * KB1 * 64 * 8, 0);
  for (int mt = 0; mt < 8; ++mt)
    for (int kb = 0; kb < KB1; ++kb)
      for (int l = 0; l < 64; ++l)
        for (int i = 0; i < 8; ++i) {
          const int m = mt * 16 + l % 16, k = kb * 32 + 8 * (l / 16) + i;
          const int j = m >> 1, po = m & 1, q = k >> 1, pi = k & 1;
          double v = 0.0;
          if (q < 2 * m1) {
            const int kx = q < m1 ? q : H - 2 * m1 + q;
            double cs, sn;
            cos_sin_2pi((long)kx * j, H, cs, sn);
            v = po == 0 ? (pi == 0 ? cs : -sn) : (pi == 0 ? sn : cs);
          }
          ef[(((size_t)mt * KB1 + kb) * 64 + l) * 8 + i] = v;
        }
}

static int ceil_log2(int v) {
  int e = 0;
  while ((1 << e) < v) ++e;
  return e;
}

}  // namespace

struct fno_plan_s {
  int ndim = 0, B = 0, Ci = 0, Co = 0;
  int grid[3] = {0, 0, 0};
  int modes[3] = {0, 0, 0};
  int dtype = 0, device = 0;
  int K = 0;            // retained modes per plane
  // plane transform (2D: axes H, W; 3D: axes Y, Z of every x-slab)
  int pH = 0, pW = 0, pm1 = 0, pm2 = 0, pMP = 0, rpt = 2, rc = 1, ppw_f = 1, ppw_i = 1;
  size_t lds_fwd = 0, lds_inv = 0;
  // 3D outer axis
  int xN = 0, xm = 0, xMP = 0;
  size_t lds_axis = 0;
  int bb = 1, split = 1;
  bool cmx = false;  // fp16 / bf16 contraction on bf16 matrix cores
  // half exchange of the forward layer: the spectra between its launches as
  // fp16 pairs with power-of-two exponents (fp16 / bf16 2D plans on the
  // matrix-core planes and contraction); the backward keeps complex fp32
  bool hx = false;
  int *xe = nullptr;           // [B][Ci] exponents of the forward spectra
  signed char *ye = nullptr;   // [B][Co][ceil(K / 4)] exponents of the contracted spectra
  // half exchange in the backward as well (fp16 hx plans whose adjoint runs
  // on the matrix-core contraction, which then multiplies fp16 operands
  // directly; bf16 plans measured no faster with it): exponents of the
  // spectra of dL/dy and of the adjoint-contracted spectra
  bool hx_b = false;
  int *ge = nullptr;           // [B][Co]
  signed char *gxe = nullptr;  // [B][Ci][ceil(K / 4)]
  // backward: the adjoint contraction (Co -> Ci channels), the weight
  // gradient, plane transforms over the other channel count (forward of g
  // over Co channels, inverse over Ci)
  int bb_a = 1, split_a = 1;
  bool cmx_a = false;
  // fp32 plans: the adjoint contraction reads W in its forward layout (no
  // conjugate-transposed copy, no W^H buffer)
  bool adj_w = false;
  bool adj_mx = false;  // the matrix-core adjoint contraction reads W itself (no W^H)
  int ppw_fg = 1, ppw_ib = 1;
  size_t lds_fg = 0, lds_ib = 0;
  int mx_grid_fg = 0, mx_grid_ib = 0;
  int mx_grid_fb = 0;  // forward planes of x and dL/dy in one launch (2D backward)
  void *wh = nullptr;  // conjugate-transposed weights [K][Co][Ci][2], storage dtype
  // row stage on MFMA (fp16 / bf16 storage, planes with H >= 64, W >= 64)
  bool mx = false;
  int mx_nt = 0, mx_mt = 0, mx_nn = 0, mx_kb1 = 0, mx_lgW = 0, mx_lg4m1 = 0, mx_grid_f = 0, mx_grid_i = 0;
  uint4 *tf = nullptr, *tb = nullptr, *ef_f = nullptr, *ef_i = nullptr;
  uint4 *tf_lo = nullptr, *tb_lo = nullptr, *ef_f_lo = nullptr, *ef_i_lo = nullptr;  // fp32 plans
  float2 *tw_h = nullptr, *tw_w = nullptr, *tw_x = nullptr;
  float2 *xh = nullptr, *yh = nullptr, *tbuf = nullptr;
  // single-launch layer (2D): variant, availability, current launch shape,
  // co-resident grid, LDS, barrier words (in the workspace)
  FusedShape fshape{};
  bool fused_ok = false;
  int shape = FNO_LAUNCH_SEPARATE;
  int fused_grid = 0;
  size_t lds_fused = 0;
  FusedBarrier *bar = nullptr;
  // FNO block (fno_block2d): Z rows between the column and row stages, the
  // planes' scale exponents, allocated by fno_block2d_prepare
  void *blk_mem = nullptr;
  uint16_t *zbuf = nullptr;
  signed char *zexp = nullptr;
  int cols_grid = 0;
  void *mem = nullptr;
  size_t ws_bytes = 0;
  std::vector<int> launches;      // the current launch shape's launches
  std::vector<int> sep_launches;  // the stand-alone kernels' sequence
};

static void set_launches(fno_plan_s &p) {
  p.launches = p.shape == FNO_LAUNCH_SEPARATE ? p.sep_launches : std::vector<int>{L_FUSED};
}

static fno_status_t map_err(hipError_t e) {
  if (e == hipSuccess) return FNO_OK;
  if (e == hipErrorOutOfMemory) return FNO_ERR_OUT_OF_MEMORY;
  return FNO_ERR_DEVICE;
}

// Validate sizes; fills the shape fields. No HIP calls.
static fno_status_t validate(fno_plan_s &p, int ndim, int batch, int c_in, int c_out, const int *grid,
                             const int *modes, fno_dtype_t dtype) {
  if (ndim != 2 && ndim != 3) return FNO_ERR_INVALID_ARG;
  if (!grid || !modes) return FNO_ERR_INVALID_ARG;
  if (batch < 1 || c_in < 1 || c_out < 1) return FNO_ERR_INVALID_ARG;
  if (batch > 65535 || c_in > 65535 || c_out > 65535) return FNO_ERR_UNSUPPORTED;
  if (dtype != FNO_F32 && dtype != FNO_F16 && dtype != FNO_BF16) return FNO_ERR_INVALID_ARG;
  for (int d = 0; d < ndim; ++d) {
    if (grid[d] < 2) return FNO_ERR_INVALID_ARG;
    if (modes[d] < 1 || modes[d] > grid[d] / 2) return FNO_ERR_INVALID_ARG;
  }
  for (int d = 0; d < ndim; ++d) {
    if (!is_pow2(grid[d]) || grid[d] < kMinAxis || grid[d] > kMaxAxis) return FNO_ERR_UNSUPPORTED;
  }
  p.ndim = ndim;
  p.B = batch;
  p.Ci = c_in;
  p.Co = c_out;
  p.dtype = (int)dtype;
  for (int d = 0; d < ndim; ++d) {
    p.grid[d] = grid[d];
    p.modes[d] = modes[d];
  }
  const int o = ndim - 2;  // plane axes are the last two
  p.pH = grid[o];
  p.pW = grid[o + 1];
  p.pm1 = modes[o];
  p.pm2 = modes[o + 1];
  p.pMP = next_pow2(p.pm1 > p.pm2 ? p.pm1 : p.pm2);
  if (p.pMP < 2) p.pMP = 2;
  const int pmin = p.pH < p.pW ? p.pH : p.pW;
  if (p.pMP > kMaxRegFFT || p.pMP > pmin / 2) return FNO_ERR_UNSUPPORTED;
  if (ndim == 3) {
    p.xN = grid[0];
    p.xm = modes[0];
    p.xMP = next_pow2(p.xm);
    if (p.xMP < 2) p.xMP = 2;
    if (p.xMP > kMaxRegFFT || p.xMP > p.xN / 2) return FNO_ERR_UNSUPPORTED;
    p.K = 4 * modes[0] * modes[1] * modes[2];
  } else {
    p.K = 2 * modes[0] * modes[1];
  }
  // plane and element counts in 64 bits, checked before any use: batch and
  // channels may each be up to 65535, whose product overflows an int
  long pts = 1;
  for (int d = 0; d < ndim; ++d) pts *= grid[d];
  const long cmax = c_in > c_out ? c_in : c_out;
  const long planes = (long)batch * cmax * (ndim == 3 ? grid[0] : 1);
  if (planes > 0x7fffffffL || (double)batch * cmax * (double)pts > 1e12) return FNO_ERR_UNSUPPORTED;
  const int np_f = (int)((long)batch * c_in * (ndim == 3 ? grid[0] : 1));
  const int np_i = (int)((long)batch * c_out * (ndim == 3 ? grid[0] : 1));
  p.rpt = plane_rpt(p.pMP, p.pW / p.pMP);
  p.rc = plane_rc(p.pH, p.pMP);
  p.ppw_f = plane_ppw(true, p.pH, p.pW, p.pm1, p.pm2, p.pMP, np_f);
  p.ppw_i = plane_ppw(false, p.pH, p.pW, p.pm1, p.pm2, p.pMP, np_i);
  p.lds_fwd = plane_fwd_lds_bytes(p.pH, p.pW, p.pm1, p.pm2, p.pMP, p.ppw_f);
  p.lds_inv = plane_inv_lds_bytes(p.pH, p.pW, p.pm1, p.pm2, p.pMP, p.ppw_i);
  p.mx = mx_supported(p.pH, p.pW, p.pm1, p.pm2, (int)dtype);
  if (p.mx) {
    p.mx_nt = mx_ntiles(p.pm2);
    p.mx_mt = (p.pm1 + 3) / 4;
    p.mx_nn = (p.pm2 + 15) / 16;
    p.mx_kb1 = (p.pm1 + 7) / 8;
    p.mx_lgW = ceil_log2(p.pW);
    p.mx_lg4m1 = ceil_log2(4 * p.pm1);
    p.lds_fwd = mx_fwd_lds_bytes(p.pH, p.pW, (int)dtype);
    p.lds_inv = mx_inv_lds_bytes(p.pH, p.pW, p.pm1, p.pm2, (int)dtype);
  }
  if (p.lds_fwd > kMaxLds || p.lds_inv > kMaxLds) return FNO_ERR_UNSUPPORTED;
  if (ndim == 3) {
    p.lds_axis = axis_fwd_lds_bytes(p.xN, p.xm, p.xMP);
    if (p.lds_axis > kMaxLds) return FNO_ERR_UNSUPPORTED;
    if ((long)batch * (c_in > c_out ? c_in : c_out) > 65535) return FNO_ERR_UNSUPPORTED;
  }
  p.bb = contract_pick_bb(batch, c_out, p.K);
  p.split = contract_pick_split(batch, c_in, c_out, p.K, p.bb);
  // The matrix-core contraction gives each workgroup a block of 8 modes x
  // 16 or 32 batch rows x 32 output channels. With fewer blocks than the
  // 256 compute units it leaves most of the chip idle, and below 16 batch
  // rows its tiles are mostly padding; there the per-mode kernel (one wave
  // per 16 modes, channels split over waves) is faster. Measured on the
  // 256x256, 64-channel layer (modes 32): 9.3 vs 20.3 us at batch 1, 17.4
  // vs 23.2 at 8, 28.2 vs 25.7 at 16, 71.8 vs 31.9 at 32.
  p.cmx = contract_mx_supported((int)dtype, c_out, p.K) && contract_mx_workgroups(batch, c_out, p.K) >= 256 &&
          batch >= 16;
  p.hx = dtype != FNO_F32 && ndim == 2 && p.mx && p.cmx;
  p.bb_a = contract_pick_bb(batch, c_in, p.K);
  p.split_a = contract_pick_split(batch, c_out, c_in, p.K, p.bb_a);
  p.cmx_a = contract_mx_supported((int)dtype, c_in, p.K) && contract_mx_workgroups(batch, c_in, p.K) >= 256 &&
            batch >= 16;
  p.adj_w = !p.cmx_a && contract_adj_supported((int)dtype, c_out, p.bb_a);
  p.adj_mx = p.cmx_a && contract_mx_wt_supported(c_out);
  // (the weight gradient reads the half-exchanged spectra 4 modes at a time)
  p.hx_b = p.hx && p.cmx_a && gradw_hx_supported((int)dtype, p.K, c_in, c_out);
  p.ppw_fg = plane_ppw(true, p.pH, p.pW, p.pm1, p.pm2, p.pMP, np_i);
  p.ppw_ib = plane_ppw(false, p.pH, p.pW, p.pm1, p.pm2, p.pMP, np_f);
  p.lds_fg = p.mx ? p.lds_fwd : plane_fwd_lds_bytes(p.pH, p.pW, p.pm1, p.pm2, p.pMP, p.ppw_fg);
  p.lds_ib = p.mx ? p.lds_inv : plane_inv_lds_bytes(p.pH, p.pW, p.pm1, p.pm2, p.pMP, p.ppw_ib);
  if (p.lds_fg > kMaxLds || p.lds_ib > kMaxLds) return FNO_ERR_UNSUPPORTED;
  if (ndim == 2) {
    p.sep_launches = {L_FWD_PLANE, L_CONTRACT, L_INV_PLANE};
  } else {
    p.sep_launches = {L_FWD_PLANE, L_FWD_AXIS, L_CONTRACT, L_INV_AXIS, L_INV_PLANE};
  }
  // the single launch: 2D only, for the plane variants it is built for
  if (ndim == 2) {
    p.fshape = FusedShape{p.mx, (int)dtype, p.pW, p.pm1, p.pm2, p.pMP, c_out};
    p.fused_ok = fused_supported(p.fshape);
    p.lds_fused = fused_lds_bytes(p.fshape, p.lds_fwd, p.lds_inv);
    if (p.lds_fused > kMaxLds) p.fused_ok = false;
  }
  // three launches by default: measured faster than the single launch at
  // every size it exists for (the cooperative launch alone costs ~19 us)
  p.shape = FNO_LAUNCH_SEPARATE;
  set_launches(p);
  return FNO_OK;
}

struct DeviceGuard {
  int prev = -1;
  hipError_t err = hipSuccess;
  explicit DeviceGuard(int dev) {
    err = hipGetDevice(&prev);
    if (err == hipSuccess && prev != dev) err = hipSetDevice(dev);
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

extern "C" {

const char *fno_status_string(fno_status_t s) {
  switch (s) {
    case FNO_OK: return "FNO_OK";
    case FNO_ERR_INVALID_ARG: return "FNO_ERR_INVALID_ARG";
    case FNO_ERR_UNSUPPORTED: return "FNO_ERR_UNSUPPORTED";
    case FNO_ERR_OUT_OF_MEMORY: return "FNO_ERR_OUT_OF_MEMORY";
    case FNO_ERR_DEVICE: return "FNO_ERR_DEVICE";
  }
  return "FNO_ERR_UNKNOWN";
}

fno_status_t fno_plan_destroy(fno_plan_t plan) {
  if (!plan) return FNO_OK;
  fno_status_t st = FNO_OK;
  if (plan->mem || plan->blk_mem) {
    DeviceGuard g(plan->device);
    if (g.err != hipSuccess) st = FNO_ERR_DEVICE;
    if (hipDeviceSynchronize() != hipSuccess) st = FNO_ERR_DEVICE;
    if (plan->mem && hipFree(plan->mem) != hipSuccess) st = FNO_ERR_DEVICE;
    if (plan->blk_mem && hipFree(plan->blk_mem) != hipSuccess) st = FNO_ERR_DEVICE;
  }
  delete plan;
  return st;
}

fno_status_t fno_plan_create(fno_plan_t *out, int ndim, int batch, int c_in, int c_out, const int *grid,
                             const int *modes, fno_dtype_t dtype, int device) {
  if (!out) return FNO_ERR_INVALID_ARG;
  *out = nullptr;
  fno_plan_s *p = new (std::nothrow) fno_plan_s();
  if (!p) return FNO_ERR_OUT_OF_MEMORY;
  fno_status_t st = validate(*p, ndim, batch, c_in, c_out, grid, modes, dtype);
  if (st != FNO_OK) {
    delete p;
    return st;
  }
  if (device < 0) {
    delete p;
    return FNO_ERR_INVALID_ARG;
  }
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess) {
    delete p;
    return FNO_ERR_DEVICE;
  }
  if (device >= ndev) {
    delete p;
    return FNO_ERR_INVALID_ARG;
  }
  p->device = device;
  DeviceGuard g(device);
  if (g.err != hipSuccess) {
    delete p;
    return FNO_ERR_DEVICE;
  }

  // workspace layout (each piece 256-byte aligned)
  auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
  const size_t n_xh = (size_t)p->B * p->Ci * p->K, n_yh = (size_t)p->B * p->Co * p->K;
  size_t n_t = 0;
  if (ndim == 3) {
    const size_t C = (size_t)2 * p->modes[1] * p->modes[2];
    n_t = (size_t)p->B * (p->Ci > p->Co ? p->Ci : p->Co) * p->xN * C;
  }
  const int nth = p->pH, ntw = p->pW, ntx = ndim == 3 ? p->xN : 0;
  size_t off = 0;
  const size_t o_th = off; off += al(nth * sizeof(float2));
  const size_t o_tw = off; off += al(ntw * sizeof(float2));
  const size_t o_tx = off; off += al(ntx * sizeof(float2));
  const size_t o_xh = off; off += al(n_xh * sizeof(float2));
  const size_t o_yh = off; off += al(n_yh * sizeof(float2));
  const size_t o_t = off; off += al(n_t * sizeof(float2));
  const bool need_wh = !p->adj_w && !p->adj_mx;
  const size_t o_wh = off; off += al(need_wh ? (size_t)p->K * p->Ci * p->Co * 2 * (p->dtype == FNO_F32 ? 4 : 2) : 0);
  const size_t o_bar = off; off += al(sizeof(FusedBarrier));
  const size_t o_xe = off; off += al(p->hx ? (size_t)p->B * p->Ci * sizeof(int) : 0);
  const size_t o_ye = off; off += al(p->hx ? (size_t)p->B * p->Co * ((p->K + 3) / 4) : 0);
  const size_t o_ge = off; off += al(p->hx_b ? (size_t)p->B * p->Co * sizeof(int) : 0);
  const size_t o_gxe = off; off += al(p->hx_b ? (size_t)p->B * p->Ci * ((p->K + 3) / 4) : 0);
  std::vector<uint16_t> tfh, tfl, tbh, tbl, efh, efl, eih, eil;
  if (p->mx) {
    const bool sp = p->dtype == FNO_F32;
    std::vector<double> v;
    fwd_fragments(p->pW, p->pm2, p->mx_nt, v);
    half_parts(v, tfh, sp ? &tfl : nullptr);
    inv_fragments(p->pW, p->pm2, p->mx_nn, v);
    half_parts(v, tbh, sp ? &tbl : nullptr);
    fwd_col_fragments(p->pH, p->pm1, p->mx_mt, v);
    half_parts(v, efh, sp ? &efl : nullptr);
    inv_col_fragments(p->pH, p->pm1, p->mx_kb1, v);
    half_parts(v, eih, sp ? &eil : nullptr);
  }
  // fragment tables: hi parts, then (fp32) lo parts, each 256-byte aligned
  std::vector<uint16_t> *tabs[8] = {&tfh, &tbh, &efh, &eih, &tfl, &tbl, &efl, &eil};
  size_t o_tab[8];
  for (int t = 0; t < 8; ++t) {
    o_tab[t] = off;
    off += al(tabs[t]->size() * 2);
  }
  p->ws_bytes = off;
  hipError_t e = hipMalloc(&p->mem, off);
  if (e != hipSuccess) {
    p->mem = nullptr;
    delete p;
    (void)hipGetLastError();
    return e == hipErrorOutOfMemory ? FNO_ERR_OUT_OF_MEMORY : FNO_ERR_DEVICE;
  }
  char *base = (char *)p->mem;
  p->tw_h = (float2 *)(base + o_th);
  p->tw_w = (float2 *)(base + o_tw);
  p->tw_x = ntx ? (float2 *)(base + o_tx) : nullptr;
  p->xh = (float2 *)(base + o_xh);
  p->yh = (float2 *)(base + o_yh);
  p->tbuf = n_t ? (float2 *)(base + o_t) : nullptr;
  p->wh = need_wh ? base + o_wh : nullptr;
  p->bar = (FusedBarrier *)(base + o_bar);
  p->xe = p->hx ? (int *)(base + o_xe) : nullptr;
  p->ye = p->hx ? (signed char *)(base + o_ye) : nullptr;
  p->ge = p->hx_b ? (int *)(base + o_ge) : nullptr;
  p->gxe = p->hx_b ? (signed char *)(base + o_gxe) : nullptr;
  uint4 *tab_ptr[8] = {};
  for (int t = 0; t < 8; ++t) tab_ptr[t] = tabs[t]->empty() ? nullptr : (uint4 *)(base + o_tab[t]);
  p->tf = tab_ptr[0];
  p->tb = tab_ptr[1];
  p->ef_f = tab_ptr[2];
  p->ef_i = tab_ptr[3];
  p->tf_lo = tab_ptr[4];
  p->tb_lo = tab_ptr[5];
  p->ef_f_lo = tab_ptr[6];
  p->ef_i_lo = tab_ptr[7];

  std::vector<float2> th = twiddles(nth), tw = twiddles(ntw);
  e = hipMemset(p->bar, 0, sizeof(FusedBarrier));
  if (e == hipSuccess) e = hipMemcpy(p->tw_h, th.data(), nth * sizeof(float2), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(p->tw_w, tw.data(), ntw * sizeof(float2), hipMemcpyHostToDevice);
  if (e == hipSuccess && ntx) {
    std::vector<float2> tx = twiddles(ntx);
    e = hipMemcpy(p->tw_x, tx.data(), ntx * sizeof(float2), hipMemcpyHostToDevice);
  }
  if (e == hipSuccess && p->mx) {
    for (int t = 0; t < 8 && e == hipSuccess; ++t)
      if (tab_ptr[t]) e = hipMemcpy(tab_ptr[t], tabs[t]->data(), tabs[t]->size() * 2, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = mx_prepare(true, p->pW, p->pm1, p->pm2, p->dtype, p->lds_fwd);
    if (e == hipSuccess) e = mx_prepare(false, p->pW, p->pm1, p->pm2, p->dtype, p->lds_inv);
    if (e == hipSuccess)
      e = mx_grid(true, p->pW, p->pm1, p->pm2, p->dtype, p->lds_fwd, p->device, p->B * p->Ci * (ndim == 3 ? p->xN : 1),
                  &p->mx_grid_f);
    if (e == hipSuccess)
      e = mx_grid(false, p->pW, p->pm1, p->pm2, p->dtype, p->lds_inv, p->device, p->B * p->Co * (ndim == 3 ? p->xN : 1),
                  &p->mx_grid_i);
    if (e == hipSuccess)
      e = mx_grid(true, p->pW, p->pm1, p->pm2, p->dtype, p->lds_fwd, p->device, p->B * p->Co * (ndim == 3 ? p->xN : 1),
                  &p->mx_grid_fg);
    if (e == hipSuccess)
      e = mx_grid(false, p->pW, p->pm1, p->pm2, p->dtype, p->lds_inv, p->device, p->B * p->Ci * (ndim == 3 ? p->xN : 1),
                  &p->mx_grid_ib);
    if (e == hipSuccess && ndim == 2 && (long)p->B * (p->Ci + p->Co) <= 0x7fffffffL)
      e = mx_grid(true, p->pW, p->pm1, p->pm2, p->dtype, p->lds_fwd, p->device, p->B * (p->Ci + p->Co), &p->mx_grid_fb,
                  true);
    if (e == hipSuccess && ndim == 2) e = mx_prepare(true, p->pW, p->pm1, p->pm2, p->dtype, p->lds_fwd, true);
  } else {
    // one kernel serves both channel counts: allow the larger LDS of the two
    if (e == hipSuccess) e = plane_prepare(true, p->pMP, p->rpt, p->dtype, std::max(p->lds_fwd, p->lds_fg));
    if (e == hipSuccess) e = plane_prepare(false, p->pMP, p->rpt, p->dtype, std::max(p->lds_inv, p->lds_ib));
  }
  if (e == hipSuccess && ndim == 3) e = axis_fwd_prepare(p->xMP, p->lds_axis);
  // the forward and the adjoint contraction may be one kernel: every
  // non-matrix-core variant is allowed the larger LDS of the two
  const size_t lds_c = std::max(p->cmx ? 0 : contract_lds_bytes(p->bb, p->split),
                                p->cmx_a ? 0 : contract_lds_bytes(p->bb_a, p->split_a));
  if (e == hipSuccess) e = p->cmx ? contract_mx_prepare(p->dtype, p->B) : contract_prepare(p->bb, p->dtype, p->Co, lds_c);
  if (e == hipSuccess)
    e = p->cmx_a ? contract_mx_prepare(p->dtype, p->B) : contract_prepare(p->bb_a, p->dtype, p->Ci, lds_c);
  if (e == hipSuccess && p->adj_w) e = contract_adj_prepare(p->bb_a, p->split_a);
  if (e == hipSuccess && p->fused_ok) {
    // the largest co-resident grid, trimmed to the most work units of a phase
    int cap = 0;
    const hipError_t ef = fused_prepare(p->fshape, p->lds_fused, p->device, &cap);
    if (ef == hipSuccess) {
      const long planes = (long)p->B * std::max(p->Ci, p->Co);
      const long units_p = p->mx ? planes : (planes + std::min(p->ppw_f, p->ppw_i) - 1) / std::min(p->ppw_f, p->ppw_i);
      const long units_c = (long)((p->K + 15) / 16) * ((p->B + 3) / 4) * ((p->Co + 15) / 16);
      p->fused_grid = (int)std::min<long>(cap, std::max(units_p, units_c));
    } else if (ef == hipErrorNotSupported) {
      p->fused_ok = false;  // no cooperative launch on this device: three launches
      p->shape = FNO_LAUNCH_SEPARATE;
      set_launches(*p);
    } else {
      e = ef;
    }
  }
  if (e != hipSuccess) {
    (void)hipFree(p->mem);
    delete p;
    return map_err(e);
  }
  *out = p;
  return FNO_OK;
}

}  // extern "C"

static size_t elem_bytes(int dtype) { return dtype == FNO_F32 ? 4 : 2; }

static bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

static fno_status_t check_exec(fno_plan_t p, int ndim, const void *x, const void *w, void *y) {
  if (!p || p->ndim != ndim) return FNO_ERR_INVALID_ARG;
  if (!x || !w || !y) return FNO_ERR_INVALID_ARG;
  if (((uintptr_t)x | (uintptr_t)w | (uintptr_t)y) & 15) return FNO_ERR_INVALID_ARG;
  size_t pts = 1;
  for (int d = 0; d < p->ndim; ++d) pts *= (size_t)p->grid[d];
  const size_t es = elem_bytes(p->dtype);
  const size_t nx = (size_t)p->B * p->Ci * pts * es, ny = (size_t)p->B * p->Co * pts * es;
  const size_t nw = (size_t)p->K * p->Ci * p->Co * 2 * es;
  if (overlap(x, nx, y, ny) || overlap(w, nw, y, ny)) return FNO_ERR_INVALID_ARG;
  return FNO_OK;
}

// Device buffers the launches exchange data through: the forward and
// contracted spectra and, in 3D, the slab transforms between the plane and
// the outer-axis passes. The plan's own workspace normally; the library's
// static scratch array for fno_spectral_conv_noalloc.
struct Bufs {
  float2 *xh, *yh, *tbuf;
  int *xe;          // half exchange: exponents of the forward spectra (fp16 pairs in xh)
  signed char *ye;  // and of the contracted spectra (fp16 pairs in yh)
};

static Bufs plan_bufs(fno_plan_t p) { return {p->xh, p->yh, p->tbuf, p->xe, p->ye}; }

// Launch helpers, parameterised by source, channel count and destination so
// the forward and the backward pass share them. nchan is Ci or Co; the
// persistent grid and planes-per-workgroup were sized for that count.

// Argument blocks of the launches, shared by the stand-alone kernels and the
// single-launch layer.

// matrix-core forward planes of `nchan` channels: 2D x -> spectra dst; 3D slabs -> tbuf
static PlaneMxFwdArgs mx_fwd_args(fno_plan_t p, const Bufs &b, const void *x, int nchan, float2 *dst, bool half) {
  const int nd = p->ndim;
  PlaneMxFwdArgs m;
  m.out16 = half ? reinterpret_cast<uint32_t *>(dst) : nullptr;
  m.oexp = half ? b.xe : nullptr;
  m.x = x;
  m.out = nd == 2 ? dst : b.tbuf;
  m.tw_h = p->tw_h;
  m.tf = p->tf;
  m.tf_lo = p->tf_lo;
  m.ef = p->ef_f;
  m.ef_lo = p->ef_f_lo;
  m.nplanes = p->B * nchan * (nd == 3 ? p->xN : 1);
  m.H = p->pH;
  m.W = p->pW;
  m.m1 = p->pm1;
  m.m2 = p->pm2;
  m.nt = p->mx_nt;
  m.mt = p->mx_mt;
  m.nn = p->mx_nn;
  m.lgW = p->mx_lgW;
  m.scale = nd == 2 ? 1.0f / ((float)p->pH * (float)p->pW) : 1.0f;
  m.x2 = m.x;
  m.out2 = m.out;
  m.nsplit = m.nplanes;
  m.out16_2 = m.out16;
  m.oexp2 = m.oexp;
  return m;
}

// VALU forward planes, as above
static PlaneFwdArgs valu_fwd_args(fno_plan_t p, const Bufs &b, const void *x, int nchan, float2 *dst) {
  const int nd = p->ndim;
  PlaneFwdArgs a;
  a.x = x;
  a.out = nd == 2 ? dst : b.tbuf;
  a.tw_h = p->tw_h;
  a.tw_w = p->tw_w;
  a.nplanes = p->B * nchan * (nd == 3 ? p->xN : 1);
  a.H = p->pH;
  a.W = p->pW;
  a.m1 = p->pm1;
  a.m2 = p->pm2;
  a.PH = p->pH / p->pMP;
  a.PW = p->pW / p->pMP;
  a.ppw = nchan == p->Ci ? p->ppw_f : p->ppw_fg;
  a.rc = p->rc;
  a.scale = nd == 2 ? 1.0f / ((float)p->pH * (float)p->pW) : 1.0f;
  return a;
}

// plane transforms of `nchan` channels: 2D x -> spectra dst; 3D slabs -> tbuf
static hipError_t fwd_plane_launch(fno_plan_t p, const Bufs &b, const void *x, int nchan, float2 *dst, hipStream_t s,
                                   bool half = false) {
  const bool own = nchan == p->Ci;
  if (p->mx)
    return launch_plane_mx_fwd(mx_fwd_args(p, b, x, nchan, dst, half), own ? p->mx_grid_f : p->mx_grid_fg, p->dtype,
                               p->lds_fwd, s);
  return launch_plane_fwd(valu_fwd_args(p, b, x, nchan, dst), p->pMP, p->rpt, p->dtype, own ? p->lds_fwd : p->lds_fg,
                          s);
}

// 2D matrix-core planes of x (Ci channels) and gy (Co channels) in one
// launch: spectra of x to xh, of gy to yh (half: fp16 pairs with exponents
// in xe and ge)
static hipError_t fwd_planes_both(fno_plan_t p, const Bufs &b, const void *x, const void *gy, hipStream_t s,
                                  bool half = false) {
  PlaneMxFwdArgs m;
  m.x = x;
  m.out = b.xh;
  m.x2 = gy;
  m.out2 = b.yh;
  m.nsplit = p->B * p->Ci;
  m.nplanes = p->B * (p->Ci + p->Co);
  m.out16 = half ? reinterpret_cast<uint32_t *>(b.xh) : nullptr;
  m.oexp = half ? b.xe : nullptr;
  m.out16_2 = half ? reinterpret_cast<uint32_t *>(b.yh) : nullptr;
  m.oexp2 = half ? p->ge : nullptr;
  m.tw_h = p->tw_h;
  m.tf = p->tf;
  m.tf_lo = p->tf_lo;
  m.ef = p->ef_f;
  m.ef_lo = p->ef_f_lo;
  m.H = p->pH;
  m.W = p->pW;
  m.m1 = p->pm1;
  m.m2 = p->pm2;
  m.nt = p->mx_nt;
  m.mt = p->mx_mt;
  m.nn = p->mx_nn;
  m.lgW = p->mx_lgW;
  m.scale = 1.0f / ((float)p->pH * (float)p->pW);
  return launch_plane_mx_fwd(m, p->mx_grid_fb, p->dtype, p->lds_fwd, s, true);
}

// 3D outer axis, forward: tbuf ([B nchan][X][C]) -> spectra dst, scaled 1/N
static hipError_t fwd_axis_launch(fno_plan_t p, const Bufs &b, int nchan, float2 *dst, hipStream_t s) {
  AxisArgs a;
  a.in = b.tbuf;
  a.out = dst;
  a.tw = p->tw_x;
  a.nvol = p->B * nchan;
  a.N = p->xN;
  a.m = p->xm;
  a.P = p->xN / p->xMP;
  a.C = 2 * p->modes[1] * p->modes[2];
  a.scale = 1.0f / ((float)p->grid[0] * (float)p->grid[1] * (float)p->grid[2]);
  return launch_axis_fwd(a, p->xMP, p->lds_axis, s);
}

static ContractArgs contract_args(fno_plan_t p, const Bufs &b, const float2 *in, const void *w, float2 *out,
                                  bool adjoint, bool half) {
  ContractArgs a;
  a.xh16 = half ? reinterpret_cast<const uint32_t *>(in) : nullptr;
  a.xexp = half ? b.xe : nullptr;
  a.yh16 = half ? reinterpret_cast<uint32_t *>(out) : nullptr;
  a.yexp = half ? b.ye : nullptr;
  a.xh = in;
  a.w = w;
  a.yh = out;
  a.B = p->B;
  a.Ci = adjoint ? p->Co : p->Ci;
  a.Co = adjoint ? p->Ci : p->Co;
  a.K = p->K;
  return a;
}

// contraction: forward (Ci -> Co with w) or adjoint (Co -> Ci with W^H;
// wt: w is the layer's W, read transposed by the matrix-core kernel)
static hipError_t contract_launch(fno_plan_t p, const Bufs &b, const float2 *in, const void *w, float2 *out,
                                  bool adjoint, hipStream_t s, bool half = false, bool wt = false) {
  const ContractArgs a = contract_args(p, b, in, w, out, adjoint, half);
  if (adjoint)
    return p->cmx_a ? launch_contract_mx(a, p->dtype, s, wt)
                    : launch_contract(a, p->bb_a, p->split_a, p->dtype, s);
  return p->cmx ? launch_contract_mx(a, p->dtype, s) : launch_contract(a, p->bb, p->split, p->dtype, s);
}

// 3D outer axis, inverse: spectra src ([B nchan][K]) -> tbuf
static hipError_t inv_axis_launch(fno_plan_t p, const Bufs &b, const float2 *src, int nchan, hipStream_t s) {
  AxisArgs a;
  a.in = src;
  a.out = b.tbuf;
  a.tw = p->tw_x;
  a.nvol = p->B * nchan;
  a.N = p->xN;
  a.m = p->xm;
  a.P = p->xN / p->xMP;
  a.C = 2 * p->modes[1] * p->modes[2];
  a.scale = 1.0f;
  return launch_axis_inv(a, p->xMP, s);
}

// matrix-core inverse planes of `nchan` channels: 2D spectra src -> y; 3D tbuf -> y
static PlaneMxInvArgs mx_inv_args(fno_plan_t p, const Bufs &b, const float2 *src, int nchan, void *y, bool half) {
  const int nd = p->ndim;
  PlaneMxInvArgs m;
  m.in16 = half ? reinterpret_cast<const uint32_t *>(src) : nullptr;
  m.iexp = half ? b.ye : nullptr;
  m.in = nd == 2 ? src : b.tbuf;
  m.y = y;
  m.tw_h = p->tw_h;
  m.tb = p->tb;
  m.tb_lo = p->tb_lo;
  m.ef = p->ef_i;
  m.ef_lo = p->ef_i_lo;
  m.nplanes = p->B * nchan * (nd == 3 ? p->xN : 1);
  m.H = p->pH;
  m.W = p->pW;
  m.m1 = p->pm1;
  m.m2 = p->pm2;
  m.nn = p->mx_nn;
  m.kb1 = p->mx_kb1;
  m.lg4m1 = p->mx_lg4m1;
  m.zg = nullptr;
  m.zexp = nullptr;
  m.zco = 0;
  return m;
}

// VALU inverse planes, as above
static PlaneInvArgs valu_inv_args(fno_plan_t p, const Bufs &b, const float2 *src, int nchan, void *y) {
  const int nd = p->ndim;
  PlaneInvArgs a;
  a.in = nd == 2 ? src : b.tbuf;
  a.y = y;
  a.tw_h = p->tw_h;
  a.tw_w = p->tw_w;
  a.nplanes = p->B * nchan * (nd == 3 ? p->xN : 1);
  a.H = p->pH;
  a.W = p->pW;
  a.m1 = p->pm1;
  a.m2 = p->pm2;
  a.PH = p->pH / p->pMP;
  a.PW = p->pW / p->pMP;
  a.ppw = nchan == p->Co ? p->ppw_i : p->ppw_ib;
  return a;
}

// inverse plane transforms of `nchan` channels: 2D spectra src -> y; 3D tbuf -> y
static hipError_t inv_plane_launch(fno_plan_t p, const Bufs &b, const float2 *src, int nchan, void *y, hipStream_t s,
                                   bool half = false) {
  const bool own = nchan == p->Co;
  if (p->mx)
    return launch_plane_mx_inv(mx_inv_args(p, b, src, nchan, y, half), own ? p->mx_grid_i : p->mx_grid_ib, p->dtype,
                               p->lds_inv, s);
  return launch_plane_inv(valu_inv_args(p, b, src, nchan, y), p->pMP, p->rpt, p->dtype, own ? p->lds_inv : p->lds_ib,
                          s);
}

// the whole 2D layer as one cooperative launch
static hipError_t fused_launch(fno_plan_t p, const Bufs &b, const void *x, const void *w, void *y, hipStream_t s) {
  const bool stall = p->shape == FNO_LAUNCH_FUSED_STALL_TEST;
  const unsigned nbar = (unsigned)p->fused_grid + (stall ? 1u : 0u);
  const unsigned spin = stall ? kStallTestSpin : kBarrierSpin;
  // the single launch exchanges complex fp32 spectra
  const ContractArgs c = contract_args(p, b, b.xh, w, b.yh, false, false);
  if (p->mx) {
    const FusedMxArgs a{mx_fwd_args(p, b, x, p->Ci, b.xh, false), c, mx_inv_args(p, b, b.yh, p->Co, y, false), p->bar,
                        nbar, spin};
    return launch_layer_fused(p->fshape, &a, p->fused_grid, p->lds_fused, s);
  }
  const FusedValuArgs a{valu_fwd_args(p, b, x, p->Ci, b.xh), c, valu_inv_args(p, b, b.yh, p->Co, y), p->bar, nbar,
                        spin};
  return launch_layer_fused(p->fshape, &a, p->fused_grid, p->lds_fused, s);
}

static hipError_t run_one(fno_plan_t p, const Bufs &b, int kind, const void *x, const void *w, void *y,
                          hipStream_t s) {
  switch (kind) {
    case L_FWD_PLANE: return fwd_plane_launch(p, b, x, p->Ci, b.xh, s, p->hx);
    case L_FWD_AXIS: return fwd_axis_launch(p, b, p->Ci, b.xh, s);
    case L_CONTRACT: return contract_launch(p, b, b.xh, w, b.yh, false, s, p->hx);
    case L_INV_AXIS: return inv_axis_launch(p, b, b.yh, p->Co, s);
    case L_INV_PLANE: return inv_plane_launch(p, b, b.yh, p->Co, y, s, p->hx);
    case L_FUSED: return fused_launch(p, b, x, w, y, s);
  }
  return hipErrorInvalidValue;
}

static const char *launch_name(int kind, bool mx) {
  switch (kind) {
    case L_FWD_PLANE: return mx ? "fno_fwd_plane_mx" : "fno_fwd_plane";
    case L_FWD_AXIS: return "fno_fwd_axis";
    case L_CONTRACT: return "fno_contract";
    case L_INV_AXIS: return "fno_inv_axis";
    case L_INV_PLANE: return mx ? "fno_inv_plane_mx" : "fno_inv_plane";
    case L_FUSED: return mx ? "fno_layer_fused_mx" : "fno_layer_fused";
  }
  return "?";
}

// Queue the layer's launches (or only launch `only`) with the exchange
// buffers b; the caller has checked the arguments and made the plan's
// device current.
static fno_status_t exec_with(fno_plan_t p, const Bufs &b, const void *x, const void *w, void *y, hipStream_t s,
                              int only) {
  const std::vector<int> *L = &p->launches;
  if (p->shape != FNO_LAUNCH_SEPARATE && only < 0) {
    // a cooperative launch is not recorded into a captured graph here: under
    // capture the layer is queued as its stand-alone kernels
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) return FNO_ERR_DEVICE;
    if (cs != hipStreamCaptureStatusNone) L = &p->sep_launches;
  }
  for (size_t i = 0; i < L->size(); ++i) {
    if (only >= 0 && (int)i != only) continue;
    hipError_t e = run_one(p, b, (*L)[i], x, w, y, s);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return map_err(e);
  }
  return FNO_OK;
}

static fno_status_t exec(fno_plan_t p, int ndim, const void *x, const void *w, void *y, void *stream, int only) {
  fno_status_t st = check_exec(p, ndim, x, w, y);
  if (st != FNO_OK) return st;
  DeviceGuard g(p->device);
  if (g.err != hipSuccess) return FNO_ERR_DEVICE;
  return exec_with(p, plan_bufs(p), x, w, y, (hipStream_t)stream, only);
}

// ---- allocation-free execution ------------------------------------------
// The exchange buffers of fno_spectral_conv_noalloc live in this file-scope
// device array. Every GPU the library runs on holds its own copy, at its own
// address, until the process ends. In host code `scratch` names a host-side
// stand-in, not device memory: its device address is looked up once per
// device (hipGetSymbolAddress with that device current) and only that
// address is ever passed to kernels.
static __device__ __align__(256) unsigned char scratch[FNO_NOALLOC_SCRATCH_BYTES];

// device address of `scratch` on `dev` (which must be current), looked up
// on the first call for that device
static hipError_t scratch_address(int dev, unsigned char **out) {
  static std::mutex mu;
  static std::map<int, unsigned char *> addr;
  std::lock_guard<std::mutex> lock(mu);
  auto it = addr.find(dev);
  if (it != addr.end()) {
    *out = it->second;
    return hipSuccess;
  }
  unsigned char *ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress((void **)&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (!ptr) return hipErrorInvalidSymbol;
  addr[dev] = ptr;
  *out = ptr;
  return hipSuccess;
}

// the plan's exchange buffers carved out of a region at `base` (NULL: only
// count); returns the bytes they take, each piece 256-byte aligned
static size_t carve(fno_plan_t p, unsigned char *base, Bufs *b) {
  auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
  const size_t n_xh = (size_t)p->B * p->Ci * p->K, n_yh = (size_t)p->B * p->Co * p->K;
  const size_t n_t = p->tbuf ? (size_t)p->B * (p->Ci > p->Co ? p->Ci : p->Co) * p->xN * 2 * p->modes[1] * p->modes[2] : 0;
  const size_t sb = p->hx ? 4 : sizeof(float2);  // bytes per exchanged mode
  const size_t o_xh = 0, o_yh = o_xh + al(n_xh * sb), o_t = o_yh + al(n_yh * sb);
  const size_t o_xe = o_t + al(n_t * sizeof(float2));
  const size_t o_ye = o_xe + al(p->hx ? (size_t)p->B * p->Ci * sizeof(int) : 0);
  const size_t total = o_ye + al(p->hx ? (size_t)p->B * p->Co * ((p->K + 3) / 4) : 0);
  if (base && b) {
    b->xh = (float2 *)(base + o_xh);
    b->yh = (float2 *)(base + o_yh);
    b->tbuf = n_t ? (float2 *)(base + o_t) : nullptr;
    b->xe = p->hx ? (int *)(base + o_xe) : nullptr;
    b->ye = p->hx ? (signed char *)(base + o_ye) : nullptr;
  }
  return total;
}

// Saved spectra of x (a forward that keeps them for the backward): the
// retained spectra in the exchange format the backward's weight gradient
// reads, then (half exchange) the per-plane exponents. Only where the forward
// leaves them in that same format: the half exchange in both passes, or
// complex fp32 in both.
static bool saved_ok(fno_plan_t p) { return p->hx == p->hx_b; }

static size_t saved_spectra_bytes(fno_plan_t p) {
  return (((size_t)p->B * p->Ci * p->K * (p->hx ? 4 : sizeof(float2))) + 255) & ~(size_t)255;
}

static size_t saved_bytes(fno_plan_t p) {
  return saved_spectra_bytes(p) + (p->hx ? (((size_t)p->B * p->Ci * sizeof(int)) + 255) & ~(size_t)255 : 0);
}

// Gradients: every launch is stream-ordered on `stream`; the spectra
// workspace holds forward(x) (or, with `saved`, the caller keeps them) and
// forward(g), then the adjoint-contracted spectra; wh holds W^H (plans whose
// adjoint contraction reads W directly have none).
static fno_status_t exec_backward(fno_plan_t p, int ndim, const void *x, const void *w, const void *gy, void *gx,
                                  void *gw, void *stream, const void *saved = nullptr) {
  if (!p || p->ndim != ndim) return FNO_ERR_INVALID_ARG;
  if (!gy || (!gx && !gw)) return FNO_ERR_INVALID_ARG;
  if ((gw && !x && !saved) || (gx && !w)) return FNO_ERR_INVALID_ARG;
  if (((uintptr_t)x | (uintptr_t)w | (uintptr_t)gy | (uintptr_t)gx | (uintptr_t)gw) & 15) return FNO_ERR_INVALID_ARG;
  if (((uintptr_t)saved & 255) || (saved && !saved_ok(p))) return FNO_ERR_INVALID_ARG;
  size_t pts = 1;
  for (int d = 0; d < p->ndim; ++d) pts *= (size_t)p->grid[d];
  const size_t es = elem_bytes(p->dtype);
  const size_t nx = (size_t)p->B * p->Ci * pts * es, ny = (size_t)p->B * p->Co * pts * es;
  const size_t nw = (size_t)p->K * p->Ci * p->Co * 2 * es;
  if (gx && (overlap(gx, nx, gy, ny) || (x && overlap(gx, nx, x, nx)) || overlap(gx, nx, w, nw)))
    return FNO_ERR_INVALID_ARG;
  if (gw && (overlap(gw, nw, gy, ny) || (x && overlap(gw, nw, x, nx)) || (w && overlap(gw, nw, w, nw)) ||
             (gx && overlap(gw, nw, gx, nx))))
    return FNO_ERR_INVALID_ARG;
  if (saved) {
    const size_t ns = saved_bytes(p);
    if ((gx && overlap(gx, nx, saved, ns)) || (gw && overlap(gw, nw, saved, ns))) return FNO_ERR_INVALID_ARG;
  }
  // launch-shape limits of the two backward-only kernels
  if (gw && (!gradw_supported(p->K) || (long)((p->Ci + 31) / 32) * ((p->Co + 31) / 32) > 65535 ||
             (long)((p->K + 7) / 8) * ((p->Ci + 31) / 32) * ((p->Co + 31) / 32) > 0x7fffffffL))
    return FNO_ERR_UNSUPPORTED;
  if (gx && (long)p->K * ((p->Ci + 31) / 32) * ((p->Co + 31) / 32) > 0x7fffffffL) return FNO_ERR_UNSUPPORTED;
  DeviceGuard g(p->device);
  if (g.err != hipSuccess) return FNO_ERR_DEVICE;
  hipStream_t s = (hipStream_t)stream;
  const bool d3 = ndim == 3;
  const Bufs b = plan_bufs(p);
  hipError_t e = hipSuccess;
  auto step = [&](hipError_t r) {
    if (e == hipSuccess) e = r == hipSuccess ? hipGetLastError() : r;
  };
  // half exchange: spectra of x with exponents xe, of dL/dy with ge, the
  // adjoint-contracted spectra with gxe (bg: the buffers seen with those)
  const bool hb = p->hx_b;
  Bufs bg = b;
  bg.xe = p->ge;
  bg.ye = p->gxe;
  // the spectra of x: transformed here into the workspace, or the caller's
  const bool fx = gw && !saved;
  const float2 *xs = saved ? (const float2 *)saved : p->xh;
  const int *xse = saved ? (const int *)((const unsigned char *)saved + saved_spectra_bytes(p)) : p->xe;
  if (fx && p->mx && !d3 && p->mx_grid_fb > 0) {
    step(fwd_planes_both(p, b, x, gy, s, hb));  // both plane sets, one launch
  } else {
    if (fx) {
      step(fwd_plane_launch(p, b, x, p->Ci, b.xh, s, hb));
      if (d3 && e == hipSuccess) step(fwd_axis_launch(p, b, p->Ci, b.xh, s));
    }
    if (e == hipSuccess) step(fwd_plane_launch(p, bg, gy, p->Co, b.yh, s, hb));
    if (d3 && e == hipSuccess) step(fwd_axis_launch(p, b, p->Co, b.yh, s));
  }
  if (gw && e == hipSuccess) {
    GradWArgs a;
    a.xs = xs;
    a.gs = p->yh;
    a.xs16 = hb ? reinterpret_cast<const uint32_t *>(xs) : nullptr;
    a.gs16 = hb ? reinterpret_cast<const uint32_t *>(p->yh) : nullptr;
    a.xexp = hb ? xse : nullptr;
    a.gexp = hb ? p->ge : nullptr;
    a.dw = gw;
    a.B = p->B;
    a.Ci = p->Ci;
    a.Co = p->Co;
    a.K = p->K;
    a.mlast = p->modes[ndim - 1];
    a.scale = (float)pts;
    step(launch_grad_w(a, p->dtype, s));
  }
  if (gx) {
    if (p->adj_w) {
      if (e == hipSuccess)
        step(launch_contract_adj(contract_args(p, b, p->yh, w, p->xh, true, false), p->bb_a, p->split_a, s));
    } else if (p->adj_mx) {
      if (e == hipSuccess) step(contract_launch(p, bg, p->yh, w, p->xh, true, s, hb, true));
    } else {
      if (e == hipSuccess) step(launch_conj_transpose(w, p->wh, p->K, p->Ci, p->Co, p->dtype, s));
      if (e == hipSuccess) step(contract_launch(p, bg, p->yh, p->wh, p->xh, true, s, hb));
    }
    if (d3 && e == hipSuccess) step(inv_axis_launch(p, b, p->xh, p->Ci, s));
    if (e == hipSuccess) step(inv_plane_launch(p, bg, p->xh, p->Ci, gx, s, hb));
  }
  return map_err(e);
}

// Copy between w and a module's weight layout (unpack: w -> user arrays).
static fno_status_t repack(fno_plan_t p, int layout, void *w, void *re, void *im, bool unpack, void *stream) {
  if (!p || !w || !re) return FNO_ERR_INVALID_ARG;
  if (layout != FNO_WEIGHTS_SPLIT && layout != FNO_WEIGHTS_CORNERS) return FNO_ERR_INVALID_ARG;
  if ((layout == FNO_WEIGHTS_SPLIT) != (im != nullptr)) return FNO_ERR_INVALID_ARG;
  const size_t es = elem_bytes(p->dtype);
  if (((uintptr_t)w | (uintptr_t)re | (uintptr_t)im) & (es - 1)) return FNO_ERR_INVALID_ARG;
  const size_t n = (size_t)p->K * p->Ci * p->Co;
  const size_t nw = 2 * n * es, nr = (layout == FNO_WEIGHTS_SPLIT ? n : 2 * n) * es;
  if (overlap(w, nw, re, nr) || (im && (overlap(w, nw, im, nr) || (unpack && overlap(re, nr, im, nr)))))
    return FNO_ERR_INVALID_ARG;
  WeightsArgs a{};
  a.w = w;
  a.re = re;
  a.im = im;
  a.n = (long)n;
  a.layout = layout == FNO_WEIGHTS_SPLIT ? W_SPLIT : W_CORNERS;
  a.unpack = unpack ? 1 : 0;
  a.ndim = p->ndim;
  a.Ci = p->Ci;
  a.Co = p->Co;
  a.m1 = p->modes[0];
  a.m2 = p->modes[1];
  a.m3 = p->ndim == 3 ? p->modes[2] : 1;
  a.mc = a.m1 * a.m2 * a.m3;
  DeviceGuard g(p->device);
  if (g.err != hipSuccess) return FNO_ERR_DEVICE;
  return map_err(launch_weights_repack(a, p->dtype, (hipStream_t)stream));
}

extern "C" {

fno_status_t fno_weights_pack(fno_plan_t plan, int layout, const void *src_re, const void *src_im, void *w,
                              void *stream) {
  return repack(plan, layout, w, const_cast<void *>(src_re), const_cast<void *>(src_im), false, stream);
}

fno_status_t fno_weights_unpack(fno_plan_t plan, int layout, const void *w, void *dst_re, void *dst_im,
                                void *stream) {
  return repack(plan, layout, const_cast<void *>(w), dst_re, dst_im, true, stream);
}

fno_status_t fno_spectral_conv2d(fno_plan_t plan, const void *x, const void *w, void *y, void *stream) {
  return exec(plan, 2, x, w, y, stream, -1);
}

fno_status_t fno_spectral_conv3d(fno_plan_t plan, const void *x, const void *w, void *y, void *stream) {
  return exec(plan, 3, x, w, y, stream, -1);
}

fno_status_t fno_spectral_conv2d_backward(fno_plan_t plan, const void *x, const void *w, const void *grad_y,
                                          void *grad_x, void *grad_w, void *stream) {
  return exec_backward(plan, 2, x, w, grad_y, grad_x, grad_w, stream);
}

fno_status_t fno_spectral_conv3d_backward(fno_plan_t plan, const void *x, const void *w, const void *grad_y,
                                          void *grad_x, void *grad_w, void *stream) {
  return exec_backward(plan, 3, x, w, grad_y, grad_x, grad_w, stream);
}

fno_status_t fno_plan_saved_bytes(fno_plan_t plan, size_t *bytes) {
  if (!plan || !bytes) return FNO_ERR_INVALID_ARG;
  if (!saved_ok(plan)) return FNO_ERR_UNSUPPORTED;
  *bytes = saved_bytes(plan);
  return FNO_OK;
}

fno_status_t fno_spectral_conv_forward_save(fno_plan_t plan, const void *x, const void *w, void *y, void *saved,
                                            void *stream) {
  if (!plan || !saved || ((uintptr_t)saved & 255)) return FNO_ERR_INVALID_ARG;
  if (!saved_ok(plan)) return FNO_ERR_UNSUPPORTED;
  fno_status_t st = check_exec(plan, plan->ndim, x, w, y);
  if (st != FNO_OK) return st;
  size_t pts = 1;
  for (int d = 0; d < plan->ndim; ++d) pts *= (size_t)plan->grid[d];
  const size_t es = elem_bytes(plan->dtype), ns = saved_bytes(plan);
  if (overlap(saved, ns, x, (size_t)plan->B * plan->Ci * pts * es) ||
      overlap(saved, ns, y, (size_t)plan->B * plan->Co * pts * es) ||
      overlap(saved, ns, w, (size_t)plan->K * plan->Ci * plan->Co * 2 * es))
    return FNO_ERR_INVALID_ARG;
  DeviceGuard g(plan->device);
  if (g.err != hipSuccess) return FNO_ERR_DEVICE;
  // the stand-alone kernels with the spectra of x (and their exponents) in
  // the caller's buffer: the contraction reads them from there
  Bufs b = plan_bufs(plan);
  b.xh = (float2 *)saved;
  if (plan->hx) b.xe = (int *)((unsigned char *)saved + saved_spectra_bytes(plan));
  const hipStream_t s = (hipStream_t)stream;
  for (int kind : plan->sep_launches) {
    hipError_t e = run_one(plan, b, kind, x, w, y, s);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return map_err(e);
  }
  return FNO_OK;
}

fno_status_t fno_spectral_conv_backward_saved(fno_plan_t plan, const void *saved, const void *w,
                                              const void *grad_y, void *grad_x, void *grad_w, void *stream) {
  if (!plan || (grad_w && !saved)) return FNO_ERR_INVALID_ARG;
  return exec_backward(plan, plan->ndim, nullptr, w, grad_y, grad_x, grad_w, stream, grad_w ? saved : nullptr);
}

fno_status_t fno_spectral_conv_noalloc(fno_plan_t plan, const void *x, const void *w, void *y, void *stream) {
  if (!plan) return FNO_ERR_INVALID_ARG;
  fno_status_t st = check_exec(plan, plan->ndim, x, w, y);
  if (st != FNO_OK) return st;
  if (carve(plan, nullptr, nullptr) > (size_t)FNO_NOALLOC_SCRATCH_BYTES) return FNO_ERR_UNSUPPORTED;
  DeviceGuard g(plan->device);
  if (g.err != hipSuccess) return FNO_ERR_DEVICE;
  unsigned char *base = nullptr;
  if (scratch_address(plan->device, &base) != hipSuccess) return FNO_ERR_DEVICE;
  Bufs b;
  carve(plan, base, &b);
  return exec_with(plan, b, x, w, y, (hipStream_t)stream, -1);
}

// ---- FNO block ---------------------------------------------------------

// the plan's dimensions the block path needs (2D, fp16 / bf16 planes of
// width 64 / 128 / 256 on matrix cores, at most 64 input channels)
static bool block_ok(fno_plan_t p) {
  return p->ndim == 2 && p->mx && p->pH == p->grid[0] && p->pW == p->grid[1] &&
         block_rows_supported(p->dtype, p->pW, p->Ci, p->mx_nn);
}

fno_status_t fno_block2d_prepare(fno_plan_t p) {
  if (!p) return FNO_ERR_INVALID_ARG;
  if (!block_ok(p)) return FNO_ERR_UNSUPPORTED;
  if (p->blk_mem) return FNO_OK;
  DeviceGuard g(p->device);
  if (g.err != hipSuccess) return FNO_ERR_DEVICE;
  const size_t nz = (size_t)p->B * p->pH * p->Co * 32 * p->mx_nn * sizeof(uint16_t);
  const size_t ne = (size_t)p->B * p->Co;
  int grid = 0;
  hipError_t e = mx_cols_prepare(p->pm1, p->pm2, p->dtype, p->lds_inv, p->device, p->B * p->Co, &grid);
  if (e != hipSuccess) return map_err(e);
  void *mem = nullptr;
  e = hipMalloc(&mem, nz + ne);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return map_err(e);
  }
  p->blk_mem = mem;
  p->zbuf = (uint16_t *)mem;
  p->zexp = (signed char *)mem + nz;
  p->cols_grid = grid;
  return FNO_OK;
}

fno_status_t fno_block2d(fno_plan_t p, const void *x, const void *w, const void *bypass, const void *bias, int act,
                         void *y, void *stream) {
  fno_status_t st = check_exec(p, 2, x, w, y);
  if (st != FNO_OK) return st;
  if (!bypass || (act != 0 && act != 1)) return FNO_ERR_INVALID_ARG;
  if (((uintptr_t)bypass | (uintptr_t)bias) & 1) return FNO_ERR_INVALID_ARG;
  if (!block_ok(p)) return FNO_ERR_UNSUPPORTED;
  DeviceGuard g(p->device);
  if (g.err != hipSuccess) return FNO_ERR_DEVICE;
  const hipStream_t s = (hipStream_t)stream;
  if (!p->blk_mem) {
    // allocating is not part of a captured graph: prepare first
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) return FNO_ERR_DEVICE;
    if (cs != hipStreamCaptureStatusNone) return FNO_ERR_UNSUPPORTED;
    st = fno_block2d_prepare(p);
    if (st != FNO_OK) return st;
  }
  const Bufs b = plan_bufs(p);
  // the spectra travel between the launches in the plan's exchange format
  hipError_t e = fwd_plane_launch(p, b, x, p->Ci, b.xh, s, p->hx);
  if (e == hipSuccess) e = contract_launch(p, b, b.xh, w, b.yh, false, s, p->hx);
  if (e == hipSuccess) {
    PlaneMxInvArgs m = mx_inv_args(p, b, b.yh, p->Co, nullptr, p->hx);
    m.zg = p->zbuf;
    m.zexp = p->zexp;
    m.zco = p->Co;
    e = launch_plane_mx_cols(m, p->cols_grid, p->dtype, p->lds_inv, s);
  }
  if (e == hipSuccess)
    e = launch_block_rows(p->zbuf, p->zexp, p->tb, x, bypass, bias, y, p->B, p->Ci, p->Co, p->pH, p->pW, p->mx_nn, act,
                          p->dtype, s);
  if (e == hipSuccess) e = hipGetLastError();
  return map_err(e);
}

fno_status_t fno_plan_workspace_bytes(fno_plan_t plan, size_t *bytes) {
  if (!plan || !bytes) return FNO_ERR_INVALID_ARG;
  *bytes = plan->ws_bytes;
  return FNO_OK;
}

fno_status_t fno_plan_num_launches(fno_plan_t plan, int *n) {
  if (!plan || !n) return FNO_ERR_INVALID_ARG;
  *n = (int)plan->launches.size();
  return FNO_OK;
}

fno_status_t fno_plan_launch_name(fno_plan_t plan, int index, const char **name) {
  if (!plan || !name || index < 0 || index >= (int)plan->launches.size()) return FNO_ERR_INVALID_ARG;
  *name = launch_name(plan->launches[index], plan->mx);
  return FNO_OK;
}

fno_status_t fno_plan_run_launch(fno_plan_t plan, int index, const void *x, const void *w, void *y,
                                 void *stream) {
  if (!plan || index < 0 || index >= (int)plan->launches.size()) return FNO_ERR_INVALID_ARG;
  return exec(plan, plan->ndim, x, w, y, stream, index);
}

fno_status_t fno_plan_set_launch_shape(fno_plan_t plan, int shape) {
  if (!plan) return FNO_ERR_INVALID_ARG;
  if (shape != FNO_LAUNCH_SEPARATE && shape != FNO_LAUNCH_FUSED && shape != FNO_LAUNCH_FUSED_STALL_TEST)
    return FNO_ERR_INVALID_ARG;
  if (shape != FNO_LAUNCH_SEPARATE && !plan->fused_ok) return FNO_ERR_UNSUPPORTED;
  plan->shape = shape;
  set_launches(*plan);
  return FNO_OK;
}

fno_status_t fno_plan_get_launch_shape(fno_plan_t plan, int *shape) {
  if (!plan || !shape) return FNO_ERR_INVALID_ARG;
  *shape = plan->shape;
  return FNO_OK;
}

fno_status_t fno_plan_check(fno_plan_t plan) {
  if (!plan) return FNO_ERR_INVALID_ARG;
  DeviceGuard g(plan->device);
  if (g.err != hipSuccess) return FNO_ERR_DEVICE;
  if (hipDeviceSynchronize() != hipSuccess) return FNO_ERR_DEVICE;
  FusedBarrier h{};
  if (hipMemcpy(&h, plan->bar, sizeof h, hipMemcpyDeviceToHost) != hipSuccess) return FNO_ERR_DEVICE;
  if (!h.err) return FNO_OK;
  // a barrier wait gave up: its state is unknown, start it afresh
  if (hipMemset(plan->bar, 0, sizeof(FusedBarrier)) != hipSuccess) return FNO_ERR_DEVICE;
  return FNO_ERR_DEVICE;
}

fno_status_t fno_plan_spectra(fno_plan_t plan, int which, void **ptr) {
  if (!plan || !ptr || which < 0 || which > 3) return FNO_ERR_INVALID_ARG;
  if (which >= 2 && !plan->hx) return FNO_ERR_INVALID_ARG;
  void *const v[4] = {plan->xh, plan->yh, plan->xe, plan->ye};
  *ptr = v[which];
  return FNO_OK;
}

fno_status_t fno_plan_spectra_format(fno_plan_t plan, int *half) {
  if (!plan || !half) return FNO_ERR_INVALID_ARG;
  *half = plan->hx ? 1 : 0;
  return FNO_OK;
}

}  // extern "C"
