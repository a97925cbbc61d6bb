// common.hpp - shared device helpers and kernel argument blocks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fft_reg.hpp"

namespace fno {

// storage dtype tags (values equal fno_dtype_t)
enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16 bits, round to nearest even (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// two fp32 -> packed bf16 pair (a in the low half), round to nearest even
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  bf16x2_t v;
  v.x = (__bf16)a;
  v.y = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// 2^e as an fp32 with e clamped to a range where it and 2^-e are normal
__device__ __forceinline__ float pow2f(int e) {
  e = max(-120, min(120, e));
  return __uint_as_float((uint32_t)(e + 127) << 23);
}

// Load two adjacent storage elements p[0], p[1] as fp32 (p 2-element aligned).
template <int DT>
__device__ __forceinline__ float2 load_pair(const void *base, size_t idx) {
  if constexpr (DT == DT_F32) {
    return *reinterpret_cast<const float2 *>(reinterpret_cast<const float *>(base) + idx);
  } else if constexpr (DT == DT_F16) {
    half2_t h = *reinterpret_cast<const half2_t *>(reinterpret_cast<const _Float16 *>(base) + idx);
    return make_float2((float)h.x, (float)h.y);
  } else {
    uint32_t v = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint16_t *>(base) + idx);
    return make_float2(__uint_as_float(v << 16), __uint_as_float(v & 0xffff0000u));
  }
}

// Store two adjacent elements (RNE conversion to the storage dtype).
template <int DT>
__device__ __forceinline__ void store_pair(void *base, size_t idx, float a, float b) {
  if constexpr (DT == DT_F32) {
    *reinterpret_cast<float2 *>(reinterpret_cast<float *>(base) + idx) = make_float2(a, b);
  } else if constexpr (DT == DT_F16) {
    half2_t h;
    h.x = (_Float16)a;
    h.y = (_Float16)b;
    *reinterpret_cast<half2_t *>(reinterpret_cast<_Float16 *>(base) + idx) = h;
  } else {
    uint32_t v = f32x2_to_bf16x2(a, b);
    *reinterpret_cast<uint32_t *>(reinterpret_cast<uint16_t *>(base) + idx) = v;
  }
}

// ---------------------------------------------------------------- arguments

// Forward transform of real planes: a pruned r2c DFT along the contiguous axis
// (length W, modes ky < m2) then a pruned c2c DFT along the other axis
// (length H, kx in the two corners of m1), output [plane][2*m1][m2] complex,
// multiplied by `scale`.
struct PlaneFwdArgs {
  const void *x;        // nplanes * H * W storage elements
  float2 *out;          // nplanes * 2*m1*m2
  const float2 *tw_h;   // exp(-2 pi i k / H), k < H
  const float2 *tw_w;   // exp(-2 pi i k / W), k < W
  int nplanes, H, W, m1, m2, PH, PW;
  int ppw;  // planes per workgroup
  int rc;   // residues per thread in the column stage
  float scale;
};

// Inverse of the above without scaling: [plane][2*m1][m2] complex -> real.
struct PlaneInvArgs {
  const float2 *in;
  void *y;
  const float2 *tw_h;
  const float2 *tw_w;
  int nplanes, H, W, m1, m2, PH, PW;
  int ppw;  // planes per workgroup
};

// Plane transforms as matrix-core products (H in [64, 256], W in {64, 128,
// 256} (fp32: {64, 128}), m1, m2 <= 32). Fragment tables hold 8 fp16 per lane
// in MFMA operand order; fp32 plans add the fp16 remainders (*_lo).
struct PlaneMxFwdArgs {
  const void *x;
  float2 *out;         // [nplanes][2 m1][m2] complex, times `scale`
  const float2 *tw_h;  // exp(-2 pi i k / H), k < H
  const uint4 *tf, *tf_lo;  // row DFT, A operand of the transposed product [NT][W/32][64]
  const uint4 *ef, *ef_lo;  // column DFT of a 64-row block, A operand [MT][4][64]
  int nplanes, H, W, m1, m2;
  int nt, mt, nn, lgW;  // column tiles of R, m-tiles of X, 16-wide ky tiles, log2 W
  float scale;
  // two-set variant only: planes nsplit .. nplanes - 1 come from x2 and go
  // to out2 (indices counted from nsplit)
  const void *x2;
  float2 *out2;
  int nsplit;
  // half exchange (NULL: complex fp32 to out / out2): the spectra as fp16
  // (re, im) pairs [planes][2 m1][m2], each plane scaled by 2^oexp[plane]
  // (the spectra are out16 * 2^-oexp); out16_2 / oexp2 for the second plane
  // set of the two-set variant (indices counted from nsplit)
  uint32_t *out16;
  int *oexp;
  uint32_t *out16_2;
  int *oexp2;
};

struct PlaneMxInvArgs {
  const float2 *in;    // [nplanes][2 m1][m2] complex
  void *y;
  const float2 *tw_h;  // exp(-2 pi i k / H), k < H
  const uint4 *ef, *ef_lo;  // inverse column DFT of a 64-row block, A operand [8][kb1][64]
  const uint4 *tb, *tb_lo;  // inverse row DFT, A operand of the transposed product [W/16][nn][64]
  int nplanes, H, W, m1, m2;
  int nn, kb1, lg4m1;  // 16-wide ky tiles, 32-deep blocks of 4 m1, ceil(log2(4 m1))
  // half exchange (NULL: complex fp32 from in): fp16 (re, im) pairs
  // [nplanes][K], each group of four modes scaled by 2^iexp[plane][k / 4]
  // (iexp has ceil(K / 4) entries per plane)
  const uint32_t *in16;
  const signed char *iexp;
  // column stage only (half storage): instead of y, the scaled fp16 Z rows
  // go to zg [B][H][zco][32 nn] halves (plane = b zco + o) and each plane's
  // scale exponent to zexp [nplanes] (Z = stored Z 2^-zexp)
  uint16_t *zg;
  signed char *zexp;
  int zco;
};

// Pruned c2c DFT along a strided axis: in [vol][N][C] -> out [vol][2*m][C]
// (forward, times `scale`), or the inverse out [vol][N][C] from [vol][2*m][C].
struct AxisArgs {
  const float2 *in;
  float2 *out;
  const float2 *tw;  // exp(-2 pi i k / N), k < N
  int nvol, N, m, P, C;
  float scale;
};

// Per-mode contraction: yh[b][o][k] = sum_i xh[b][i][k] w[k][i][o].
struct ContractArgs {
  const float2 *xh;  // [B][Ci][K]
  const void *w;     // [K][Ci][Co][2] storage dtype
  float2 *yh;        // [B][Co][K]
  int B, Ci, Co, K;
  // half exchange (matrix-core contraction only; used when xh16 is not
  // NULL): the spectra in the layouts of PlaneMxFwdArgs::out16 / oexp and
  // PlaneMxInvArgs::in16 / iexp
  const uint32_t *xh16;
  const int *xexp;
  uint32_t *yh16;
  signed char *yexp;
};

// Weight gradient: dw[k][i][o] = scale * gamma(k) * sum_b conj(xs[b][i][k])
// gs[b][o][k], gamma(k) = 1 when k % mlast == 0 (last-axis mode index 0),
// else 2.
struct GradWArgs {
  const float2 *xs;  // [B][Ci][K]
  const float2 *gs;  // [B][Co][K]
  // half exchange (fp16 / bf16 plans; both or neither, xs / gs unused then): fp16
  // (re, im) pairs in the same layouts, plane (b, c) scaled by 2^exp[b][c]
  const uint32_t *xs16, *gs16;
  const int *xexp, *gexp;
  void *dw;          // [K][Ci][Co][2] storage dtype
  int B, Ci, Co, K, mlast;
  float scale;
};

// Weight repacking between the layer's w and a module's layout.
enum : int { W_SPLIT = 0, W_CORNERS = 1 };
struct WeightsArgs {
  void *w;       // [K][Ci][Co][2] storage dtype
  void *re, *im; // W_SPLIT: [K][Ci][Co] each; W_CORNERS: re = [corner][Ci][Co][modes in corner][2], im unused
  long n;        // K * Ci * Co
  int layout, unpack, ndim, Ci, Co, m1, m2, m3, mc;  // mc: modes in one corner
};

// The whole 2D layer as one launch (forward planes, contraction, inverse
// planes joined by grid barriers). Barrier state lives in the plan's
// workspace: `count` workgroups arrived at the current barrier (zero between
// barriers), `gen` completed barriers, `err` set when a wait gave up; each
// on its own 128-byte line.
struct FusedBarrier {
  unsigned count, pad0[31], gen, pad1[31], err, pad2[31];
};

struct FusedValuArgs {
  PlaneFwdArgs fwd;
  ContractArgs ctr;
  PlaneInvArgs inv;
  FusedBarrier *bar;
  unsigned nbar;  // workgroups a barrier waits for (the grid size)
  unsigned spin;  // polls before a barrier wait gives up
};

struct FusedMxArgs {
  PlaneMxFwdArgs fwd;
  ContractArgs ctr;
  PlaneMxInvArgs inv;
  FusedBarrier *bar;
  unsigned nbar;
  unsigned spin;
};

// what selects the single-launch kernel variant
struct FusedShape {
  bool mx;           // matrix-core planes, else VALU planes
  int dtype, W, m1, m2, MP, Co;
};

bool fused_supported(const FusedShape &f);
size_t fused_lds_bytes(const FusedShape &f, size_t lds_fwd, size_t lds_inv);
// raises the kernel's LDS allowance and returns the largest co-resident grid
hipError_t fused_prepare(const FusedShape &f, size_t lds, int device, int *grid);
// args: FusedValuArgs or FusedMxArgs as f.mx says; a cooperative launch
hipError_t launch_layer_fused(const FusedShape &f, const void *args, int grid, size_t lds, hipStream_t s);

// Allow kernel k at least `lds` bytes of dynamic LDS. The attribute belongs
// to the kernel, not to a plan, and several live plans can share one
// kernel, so the cap only ever grows (a later, smaller plan must not lower
// it under an earlier one's launches). Kept per device (the current one).
// Thread-safe.
hipError_t raise_lds_cap(const void *k, size_t lds);

// host launchers (defined next to their kernels)
int plane_rpt(int MP, int PW);
int plane_rc(int H, int MP);
int plane_ppw(bool fwd, int H, int W, int m1, int m2, int MP, int nplanes);
size_t plane_fwd_lds_bytes(int H, int W, int m1, int m2, int MP, int ppw);
size_t plane_inv_lds_bytes(int H, int W, int m1, int m2, int MP, int ppw);
size_t axis_fwd_lds_bytes(int N, int m, int MP);
hipError_t plane_prepare(bool fwd, int MP, int rpt, int dtype, size_t lds);
hipError_t launch_plane_fwd(const PlaneFwdArgs &a, int MP, int rpt, int dtype, size_t lds, hipStream_t s);
hipError_t launch_plane_inv(const PlaneInvArgs &a, int MP, int rpt, int dtype, size_t lds, hipStream_t s);
int mx_ntiles(int m2);
bool mx_supported(int H, int W, int m1, int m2, int dtype);
size_t mx_fwd_lds_bytes(int H, int W, int dtype);
size_t mx_inv_lds_bytes(int H, int W, int m1, int m2, int dtype);
// two: the forward kernel variant that takes two plane sets (x2 / out2 / nsplit)
hipError_t mx_prepare(bool fwd, int W, int m1, int m2, int dtype, size_t lds, bool two = false);
hipError_t mx_grid(bool fwd, int W, int m1, int m2, int dtype, size_t lds, int device, int nplanes, int *grid,
                   bool two = false);
hipError_t launch_plane_mx_fwd(const PlaneMxFwdArgs &a, int grid, int dtype, size_t lds, hipStream_t s,
                               bool two = false);
hipError_t launch_plane_mx_inv(const PlaneMxInvArgs &a, int grid, int dtype, size_t lds, hipStream_t s);
int mx_fwd_waves(int W, int m1, int m2, int dtype);
hipError_t axis_fwd_prepare(int MP, size_t lds);
hipError_t launch_axis_fwd(const AxisArgs &a, int MP, size_t lds, hipStream_t s);
hipError_t launch_axis_inv(const AxisArgs &a, int MP, hipStream_t s);
int contract_pick_bb(int B, int Co, int K);
int contract_pick_split(int B, int Ci, int Co, int K, int bb);
size_t contract_lds_bytes(int bb, int S);
hipError_t contract_prepare(int bb, int dtype, int Co, size_t lds);
hipError_t launch_contract(const ContractArgs &a, int bb, int S, int dtype, hipStream_t s);
// adjoint contraction straight from W (fp32): args as the adjoint's (Ci =
// the layer's Co, the reduction; Co = the layer's Ci), w in the forward layout
bool contract_adj_supported(int dtype, int c_out, int bb);
size_t contract_adj_lds_bytes(int bb, int S);
hipError_t contract_adj_prepare(int bb, int S);
hipError_t launch_contract_adj(const ContractArgs &a, int bb, int S, hipStream_t s);
bool contract_mx_supported(int dtype, int Co, int K);
long contract_mx_workgroups(int B, int Co, int K);
size_t contract_mx_lds_bytes(int dtype, int B);
hipError_t contract_mx_prepare(int dtype, int B);
// wt: w holds the layer's W[K][Co][Ci] and the product's weight is its
// conjugate transpose (the backward's adjoint contraction); needs Ci % 4 == 0
hipError_t launch_contract_mx(const ContractArgs &a, int dtype, hipStream_t s, bool wt = false);
bool contract_mx_wt_supported(int Ci);

hipError_t launch_weights_repack(const WeightsArgs &a, int dtype, hipStream_t s);
hipError_t launch_conj_transpose(const void *w, void *wh, int K, int Ci, int Co, int dtype, hipStream_t s);
bool gradw_supported(int K);
bool gradw_hx_supported(int dtype, int K, int Ci, int Co);
hipError_t launch_grad_w(const GradWArgs &a, int dtype, hipStream_t s);

hipError_t launch_channel_mix(const void *x, const void *A, const void *bias, const void *add, void *y, int B,
                              int I, int O, long P, int act, int dtype, hipStream_t s);
hipError_t launch_projection(const void *x, const void *Q1, const void *q1, const void *Q2, const void *q2, void *y,
                             int B, int I, int J, int C, long P, int dtype, hipStream_t s);
// first block's weights with the lift folded in (see pointwise.hip)
hipError_t launch_lift_fold(const void *P, const void *p, const void *w, const void *Wb, const void *b, void *wf,
                            void *af, void *bf, int K, int J, int C, int dtype, hipStream_t s);
// inverse column stage alone (Z rows out), fp16 / bf16 planes
hipError_t mx_cols_prepare(int m1, int m2, int dtype, size_t lds, int device, int nplanes, int *grid);
hipError_t launch_plane_mx_cols(const PlaneMxInvArgs &a, int grid, int dtype, size_t lds, hipStream_t s);
// FNO block epilogue: inverse row stage of the scaled Z rows + 1x1 + bias + act
bool block_rows_supported(int dtype, int W, int Ci, int NN);
hipError_t launch_block_rows(const uint16_t *zg, const signed char *zexp, const void *tb, const void *x,
                             const void *wb, const void *bias, void *y, int B, int Ci, int Co, int H, int W, int NN,
                             int act, int dtype, hipStream_t s);
constexpr int kMixMaxIn = 128;   // channel mix: input channels
constexpr int kProjMaxIn = 64;   // projection: input channels
constexpr int kProjMaxHidden = 128;
constexpr int kProjMaxOut = 4;

}  // namespace fno

#include "bounds.hpp"
