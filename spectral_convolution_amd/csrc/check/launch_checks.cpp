// launch_checks.cpp - the bounds-check build's model of every launch (see
// bounds.hpp): per launcher, the span of each buffer its kernel touches,
// derived from the argument block the way the kernel indexes it, and the
// kernel's structural assumptions. Host code only.

#include "../plane_mfma.hpp"

#include <cstdio>

namespace fno {

namespace {

constexpr size_t kLdsMax = 160 * 1024;

size_t es_of(int dtype) { return dtype == DT_F32 ? 4 : 2; }

int ceil_lg(int v) {
  int e = 0;
  while ((1 << e) < v) ++e;
  return e;
}

struct Ctx {
  const char *name;
  void span(const char *what, const void *p, size_t n) const {
    if (n && (!p || !bounds::inside(p, n))) bounds::report(name, what);
  }
  void need(const char *what, bool ok) const {
    if (!ok) bounds::report(name, what);
  }
};

bool pow2_plane(int n) { return n == 64 || n == 128 || n == 256; }

void spans_mx_fwd(const Ctx &c, const PlaneMxFwdArgs &a, int dtype, bool two) {
  const size_t es = es_of(dtype), K = (size_t)2 * a.m1 * a.m2, px = (size_t)a.H * a.W;
  const size_t n1 = two ? (size_t)a.nsplit : (size_t)a.nplanes, n2 = (size_t)a.nplanes - n1;
  c.span("x", a.x, n1 * px * es);
  if (two) c.span("x2", a.x2, n2 * px * es);
  if (a.out16) {
    c.span("out16", a.out16, n1 * K * 4);
    c.span("oexp", a.oexp, n1 * 4);
    if (two) {
      c.span("out16_2", a.out16_2, n2 * K * 4);
      c.span("oexp2", a.oexp2, n2 * 4);
    }
  } else {
    c.span("out", a.out, n1 * K * 8);
    if (two) c.span("out2", a.out2, n2 * K * 8);
  }
  c.span("tw_h", a.tw_h, (size_t)a.H * 8);
  const size_t ntf = (size_t)a.nt * (a.W / 32) * 64 * 16, nef = (size_t)a.mt * 4 * 64 * 16;
  c.span("tf", a.tf, ntf);
  c.span("ef", a.ef, nef);
  if (dtype == DT_F32) {
    c.span("tf_lo", a.tf_lo, ntf);
    c.span("ef_lo", a.ef_lo, nef);
  }
  c.need("H in {64, 128, 256}", pow2_plane(a.H));
  c.need("W in {64, 128, 256} (fp32: 64, 128)", pow2_plane(a.W) && (dtype != DT_F32 || a.W <= 128));
  c.need("1 <= m1 <= 32, 2 m1 <= H", a.m1 >= 1 && a.m1 <= 32 && 2 * a.m1 <= a.H);
  c.need("1 <= m2 <= 32, m2 <= W / 2 + 1", a.m2 >= 1 && a.m2 <= 32 && a.m2 <= a.W / 2 + 1);
  c.need("nt = R column tiles of m2", a.nt == mx_ntiles(a.m2));
  c.need("mt = ceil(m1 / 4), one m-tile per wave", a.mt == (a.m1 + 3) / 4 && a.mt <= mx_fwd_waves(a.W, a.m1, a.m2, dtype));
  c.need("nn = ceil(m2 / 16) <= 2", a.nn == (a.m2 + 15) / 16 && a.nn <= 2);
  c.need("lgW = log2 W", (1 << a.lgW) == a.W);
}

void spans_mx_inv(const Ctx &c, const PlaneMxInvArgs &a, int dtype, bool cols) {
  const size_t es = es_of(dtype), K = (size_t)2 * a.m1 * a.m2, np = (size_t)a.nplanes;
  if (a.in16) {
    c.span("in16", a.in16, np * K * 4);
    c.span("iexp", a.iexp, np * ((K + 3) / 4));
  } else {
    c.span("in", a.in, np * K * 8);
  }
  c.span("tw_h", a.tw_h, (size_t)a.H * 8);
  const size_t nef = (size_t)8 * a.kb1 * 64 * 16, ntb = (size_t)(a.W / 16) * a.nn * 64 * 16;
  c.span("ef", a.ef, nef);
  if (dtype == DT_F32) c.span("ef_lo", a.ef_lo, nef);
  if (cols) {
    c.need("column stage: fp16 / bf16 planes", dtype != DT_F32);
    c.need("zco divides the planes", a.zco >= 1 && a.nplanes % a.zco == 0);
    c.span("zg", a.zg, np * a.H * 32 * a.nn * 2);
    c.span("zexp", a.zexp, np);
  } else {
    c.span("y", a.y, np * a.H * a.W * es);
    c.span("tb", a.tb, ntb);
    if (dtype == DT_F32) c.span("tb_lo", a.tb_lo, ntb);
  }
  c.need("H in {64, 128, 256}", pow2_plane(a.H));
  c.need("W in {64, 128, 256} (fp32: 64, 128)", pow2_plane(a.W) && (dtype != DT_F32 || a.W <= 128));
  c.need("1 <= m1 <= 32, 2 m1 <= H", a.m1 >= 1 && a.m1 <= 32 && 2 * a.m1 <= a.H);
  c.need("1 <= m2 <= 32", a.m2 >= 1 && a.m2 <= 32);
  c.need("nn = ceil(m2 / 16)", a.nn == (a.m2 + 15) / 16);
  c.need("kb1 = ceil(m1 / 8)", a.kb1 == (a.m1 + 7) / 8);
  c.need("lg4m1 = ceil(log2(4 m1))", a.lg4m1 == ceil_lg(4 * a.m1));
  const bool sm = a.m1 <= 16 && a.m2 <= 16;
  const int NY = sm ? InvGeom<true>::NY : InvGeom<false>::NY, YR = sm ? InvGeom<true>::YR : InvGeom<false>::YR;
  const int YP = sm ? InvGeom<true>::YP : InvGeom<false>::YP, ZP = sm ? InvGeom<true>::ZP : InvGeom<false>::ZP;
  const int KBM = sm ? InvGeom<true>::KBM : InvGeom<false>::KBM, NNM = sm ? InvGeom<true>::NNM : InvGeom<false>::NNM;
  c.need("k-blocks of E' Y within the geometry", a.kb1 <= KBM);
  c.need("ky tiles within the geometry", a.nn <= NNM);
  c.need("spectra rows: m2 <= YR", a.m2 <= YR);
  c.need("spectra row: 2 m1 words and the fragment reads fit YP", 4 * a.m1 <= YP && 32 * a.kb1 <= YP);
  c.need("Z row: the fragment reads fit ZP", 32 * a.nn <= ZP);
  const int nk = (a.m2 + 3) / 4, lgk = nk <= 1 ? 0 : nk <= 2 ? 1 : nk <= 4 ? 2 : 3;
  c.need("spectra tiles fit the threads' values", (((2 * a.m1 + 7) / 8) << lgk) <= 8 * NY);
}

void spans_contract(const Ctx &c, const ContractArgs &a, int dtype) {
  const size_t es = es_of(dtype), K = (size_t)a.K;
  if (a.xh16) {
    c.span("xh16", a.xh16, (size_t)a.B * a.Ci * K * 4);
    c.span("xexp", a.xexp, (size_t)a.B * a.Ci * 4);
  } else {
    c.span("xh", a.xh, (size_t)a.B * a.Ci * K * 8);
  }
  c.span("w", a.w, K * a.Ci * a.Co * 2 * es);
  if (a.yh16) {
    c.span("yh16", a.yh16, (size_t)a.B * a.Co * K * 4);
    c.span("yexp", a.yexp, (size_t)a.B * a.Co * ((K + 3) / 4));
  } else {
    c.span("yh", a.yh, (size_t)a.B * a.Co * K * 8);
  }
  c.need("half exchange both ways or neither", (a.xh16 == nullptr) == (a.yh16 == nullptr));
}

void spans_plane_fwd(const Ctx &c, const PlaneFwdArgs &a, int dtype) {
  const size_t es = es_of(dtype);
  c.span("x", a.x, (size_t)a.nplanes * a.H * a.W * es);
  c.span("out", a.out, (size_t)a.nplanes * 2 * a.m1 * a.m2 * 8);
  c.span("tw_h", a.tw_h, (size_t)a.H * 8);
  c.span("tw_w", a.tw_w, (size_t)a.W * 8);
}

void spans_plane_inv(const Ctx &c, const PlaneInvArgs &a, int dtype) {
  const size_t es = es_of(dtype);
  c.span("in", a.in, (size_t)a.nplanes * 2 * a.m1 * a.m2 * 8);
  c.span("y", a.y, (size_t)a.nplanes * a.H * a.W * es);
  c.span("tw_h", a.tw_h, (size_t)a.H * 8);
  c.span("tw_w", a.tw_w, (size_t)a.W * 8);
}

void grid_lds(const Ctx &c, int grid, int work, size_t lds, size_t need_lds) {
  c.need("grid of 1 .. work items", grid >= 1 && grid <= work);
  c.need("LDS at most 160 KiB", lds <= kLdsMax);
  c.need("LDS covers the kernel's layout", lds >= need_lds);
}

}  // namespace

void check_plane_fwd(const PlaneFwdArgs &a, int MP, int rpt, int dtype, size_t lds) {
  const Ctx c{"fno_fwd_plane"};
  (void)rpt;
  spans_plane_fwd(c, a, dtype);
  c.need("MP divides the plane", MP >= 1 && a.H % MP == 0 && a.W % MP == 0 && a.PH * MP == a.H && a.PW * MP == a.W);
  c.need("planes per workgroup >= 1", a.ppw >= 1);
  c.need("modes within the plane", 2 * a.m1 <= a.H && a.m2 <= a.W / 2 + 1 && a.m1 >= 1 && a.m2 >= 1);
  grid_lds(c, (a.nplanes + a.ppw - 1) / a.ppw, a.nplanes, lds,
           plane_fwd_lds_bytes(a.H, a.W, a.m1, a.m2, MP, a.ppw));
}

void check_plane_inv(const PlaneInvArgs &a, int MP, int rpt, int dtype, size_t lds) {
  const Ctx c{"fno_inv_plane"};
  (void)rpt;
  spans_plane_inv(c, a, dtype);
  c.need("MP divides the plane", MP >= 1 && a.H % MP == 0 && a.W % MP == 0 && a.PH * MP == a.H && a.PW * MP == a.W);
  c.need("planes per workgroup >= 1", a.ppw >= 1);
  grid_lds(c, (a.nplanes + a.ppw - 1) / a.ppw, a.nplanes, lds,
           plane_inv_lds_bytes(a.H, a.W, a.m1, a.m2, MP, a.ppw));
}

void check_plane_mx_fwd(const PlaneMxFwdArgs &a, int grid, int dtype, size_t lds, bool two) {
  const Ctx c{"fno_fwd_plane_mx"};
  spans_mx_fwd(c, a, dtype, two);
  c.need("two plane sets: 0 < nsplit < nplanes", !two || (a.nsplit > 0 && a.nsplit < a.nplanes));
  grid_lds(c, grid, a.nplanes, lds, mx_fwd_lds_bytes(a.H, a.W, dtype));
}

void check_plane_mx_inv(const PlaneMxInvArgs &a, int grid, int dtype, size_t lds, bool cols) {
  const Ctx c{cols ? "fno_inv_cols_mx" : "fno_inv_plane_mx"};
  spans_mx_inv(c, a, dtype, cols);
  grid_lds(c, grid, a.nplanes, lds, mx_inv_lds_bytes(a.H, a.W, a.m1, a.m2, dtype));
}

void check_axis(const AxisArgs &a, bool fwd) {
  const Ctx c{fwd ? "fno_fwd_axis" : "fno_inv_axis"};
  const size_t full = (size_t)a.nvol * a.N * a.C * 8, part = (size_t)a.nvol * 2 * a.m * a.C * 8;
  c.span("in", a.in, fwd ? full : part);
  c.span("out", a.out, fwd ? part : full);
  c.span("tw", a.tw, (size_t)a.N * 8);
  c.need("2 m <= N", a.m >= 1 && 2 * a.m <= a.N);
}

void check_contract(const ContractArgs &a, int dtype, bool mx) {
  const Ctx c{mx ? "fno_contract_mx" : "fno_contract"};
  spans_contract(c, a, dtype);
  if (mx) c.need("matrix-core contraction: fp16 / bf16, Co % 4 == 0, K even",
                 dtype != DT_F32 && a.Co % 4 == 0 && a.K % 2 == 0);
  else c.need("the half exchange only on the matrix-core contraction", a.xh16 == nullptr);
}

void check_contract_adj(const ContractArgs &a, int bb, int S, size_t wave_bytes, size_t stage_bytes) {
  const Ctx c{"fno_contract_adj"};
  spans_contract(c, a, DT_F32);
  c.need("fp32 spectra both ways", a.xh16 == nullptr && a.yh16 == nullptr);
  c.need("even reduction count (16-byte pairs of W)", a.Ci >= 2 && a.Ci % 2 == 0);
  c.need("batch tile of 4 or 8 rows", bb == 1 || bb == 2);
  c.need("S divides the 16 BB partial-sum pairs", S == 1 || S == 2 || S == 4 || S == 8);
  c.need("a wave's LDS share holds its staging region and its partial sums",
         wave_bytes >= stage_bytes && wave_bytes >= (size_t)bb * 16 * 2 * 64 * 4);
}

void check_grad_w(const GradWArgs &a, int dtype) {
  const Ctx c{"fno_grad_w"};
  const size_t K = (size_t)a.K;
  if (a.xs16) {
    c.span("xs16", a.xs16, (size_t)a.B * a.Ci * K * 4);
    c.span("gs16", a.gs16, (size_t)a.B * a.Co * K * 4);
    c.span("xexp", a.xexp, (size_t)a.B * a.Ci * 4);
    c.span("gexp", a.gexp, (size_t)a.B * a.Co * 4);
    c.need("half exchange: both operands, fp16 / bf16 plan, K % 4 == 0 (16-byte mode quads)",
           a.gs16 && a.xexp && a.gexp && dtype != DT_F32 && a.K % 4 == 0);
  } else {
    c.span("xs", a.xs, (size_t)a.B * a.Ci * K * 8);
    c.span("gs", a.gs, (size_t)a.B * a.Co * K * 8);
  }
  c.span("dw", a.dw, K * a.Ci * a.Co * 2 * es_of(dtype));
  c.need("last-axis modes divide K", a.mlast >= 1 && a.K % a.mlast == 0);
}

void check_conj_transpose(const void *w, const void *wh, int K, int Ci, int Co, int dtype) {
  const Ctx c{"fno_conj_transpose"};
  const size_t n = (size_t)K * Ci * Co * 2 * es_of(dtype);
  c.span("w", w, n);
  c.span("wh", wh, n);
}

void check_weights_repack(const WeightsArgs &a, int dtype) {
  const Ctx c{"fno_weights_repack"};
  const size_t es = es_of(dtype), n = (size_t)a.n;
  c.span("w", a.w, n * 2 * es);
  if (a.layout == W_SPLIT) {
    c.span("re", a.re, n * es);
    c.span("im", a.im, n * es);
  } else {
    c.span("corners", a.re, n * 2 * es);
  }
  const long K = a.ndim == 2 ? 2L * a.m1 * a.m2 : 4L * a.m1 * a.m2 * a.m3;
  c.need("n = K Ci Co", a.n == K * a.Ci * a.Co);
  c.need("modes per corner", a.mc == (a.ndim == 2 ? a.m1 * a.m2 : a.m1 * a.m2 * a.m3));
}

void check_layer_fused(const FusedShape &f, const void *args, int grid, size_t lds) {
  const Ctx c{f.mx ? "fno_layer_fused_mx" : "fno_layer_fused"};
  c.need("LDS at most 160 KiB", lds <= kLdsMax);
  c.need("a grid", grid >= 1);
  if (f.mx) {
    const FusedMxArgs &a = *static_cast<const FusedMxArgs *>(args);
    spans_mx_fwd(c, a.fwd, f.dtype, false);
    spans_contract(c, a.ctr, f.dtype);
    spans_mx_inv(c, a.inv, f.dtype, false);
    c.span("bar", a.bar, sizeof(FusedBarrier));
    c.need("barrier waits for the grid (or one more: stall test)",
           a.nbar == (unsigned)grid || a.nbar == (unsigned)grid + 1);
    c.need("LDS covers both plane layouts",
           lds >= mx_fwd_lds_bytes(a.fwd.H, a.fwd.W, f.dtype) &&
               lds >= mx_inv_lds_bytes(a.inv.H, a.inv.W, a.inv.m1, a.inv.m2, f.dtype));
  } else {
    const FusedValuArgs &a = *static_cast<const FusedValuArgs *>(args);
    spans_plane_fwd(c, a.fwd, f.dtype);
    spans_contract(c, a.ctr, f.dtype);
    spans_plane_inv(c, a.inv, f.dtype);
    c.span("bar", a.bar, sizeof(FusedBarrier));
    c.need("barrier waits for the grid (or one more: stall test)",
           a.nbar == (unsigned)grid || a.nbar == (unsigned)grid + 1);
  }
}

void check_channel_mix(const void *x, const void *A, const void *bias, const void *add, const void *y, int B, int I,
                       int O, long P, int dtype) {
  const Ctx c{"fno_channel_mix"};
  const size_t es = es_of(dtype);
  c.span("x", x, (size_t)B * I * P * es);
  c.span("A", A, (size_t)O * I * es);
  if (bias) c.span("bias", bias, (size_t)O * es);
  if (add) c.span("add", add, (size_t)B * O * P * es);
  c.span("y", y, (size_t)B * O * P * es);
  c.need("1 <= c_in <= 128", I >= 1 && I <= kMixMaxIn);
}

void check_projection(const void *x, const void *Q1, const void *q1, const void *Q2, const void *q2, const void *y,
                      int B, int I, int J, int C, long P, int dtype) {
  const Ctx c{"fno_projection"};
  const size_t es = es_of(dtype);
  c.span("x", x, (size_t)B * I * P * es);
  c.span("Q1", Q1, (size_t)J * I * es);
  c.span("q1", q1, (size_t)J * es);
  c.span("Q2", Q2, (size_t)C * J * es);
  c.span("q2", q2, (size_t)C * es);
  c.span("y", y, (size_t)B * C * P * es);
  c.need("c_in <= 64, hidden <= 128, c_out <= 4", I <= kProjMaxIn && J <= kProjMaxHidden && C <= kProjMaxOut);
}

void check_lift_fold(const void *P, const void *p, const void *w, const void *Wb, const void *b, const void *wf,
                     const void *af, const void *bf, int K, int J, int C, int dtype) {
  const Ctx c{"fno_lift_fold"};
  const size_t es = es_of(dtype);
  c.span("P", P, (size_t)C * J * es);
  c.span("p", p, (size_t)C * es);
  c.span("w", w, (size_t)K * C * C * 2 * es);
  c.span("Wb", Wb, (size_t)C * C * es);
  c.span("b", b, (size_t)C * es);
  c.span("wf", wf, (size_t)K * J * C * 2 * es);
  c.span("af", af, (size_t)C * J * es);
  c.span("bf", bf, (size_t)C * es);
  c.need("P fits the LDS stage", (long)C * J <= (long)kProjMaxIn * kMixMaxIn);
}

void check_block_rows(const void *zg, const void *zexp, const void *tb, const void *x, const void *wb,
                      const void *bias, const void *y, int B, int Ci, int Co, int H, int W, int NN, int dtype) {
  const Ctx c{"fno_block_rows"};
  const size_t es = es_of(dtype);
  c.span("zg", zg, (size_t)B * H * Co * 32 * NN * 2);
  c.span("zexp", zexp, (size_t)B * Co);
  c.span("tb", tb, (size_t)(W / 16) * NN * 64 * 16);
  c.span("x", x, (size_t)B * Ci * H * W * es);
  c.span("wb", wb, (size_t)Co * Ci * es);
  if (bias) c.span("bias", bias, (size_t)Co * es);
  c.span("y", y, (size_t)B * Co * H * W * es);
  c.need("fp16 / bf16, W in {64, 128, 256}, c_in <= 64, 1 or 2 ky tiles",
         dtype != DT_F32 && pow2_plane(W) && Ci >= 1 && Ci <= 64 && (NN == 1 || NN == 2));
}

}  // namespace fno
