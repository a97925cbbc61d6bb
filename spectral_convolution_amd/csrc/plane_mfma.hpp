// plane_mfma.hpp - plane transforms of fp16 / bf16 / fp32 planes as two
// streamed matrix-core contractions each way (device bodies, shared by the
// stand-alone kernels and the single-launch layer).
//
// The layer keeps m2 of the W/2+1 row frequencies and 2 m1 of the H column
// frequencies (TurboFNO write-up, sections 2.1 and 3.1: truncation means the
// FFT only has to produce, or consume, a few modes). Each one-dimensional
// transform is therefore a thin dense product:
//
//   forward  R[h][c]   = sum_w x[h][w] T[w][c]          (c = 2 ky + re/im)
//            X[q][ky]  = sum_h e^{-2 pi i kx(q) h / H} R[h][ky]
//   inverse  Z[h][ky]  = sum_q e^{+2 pi i kx(q) h / H} Y[q][ky]
//            y[h][w]   = sum_c Z[h][c] T'[c][w]
//
// with T[w][2ky] = cos(2 pi ky w / W), T[w][2ky+1] = -sin(..), and T'
// carrying the c2r weights (1 for ky = 0, whose imaginary part drops out, 2
// otherwise). kx(q) = q for q < m1 and H - 2 m1 + q above (the two corners).
// All four run on v_mfma_f32_16x16x32_f16 with fp32 accumulation.
//
// Rows are streamed in rounds of 64. The column product of one round uses
// the same 64-row twiddle block for every round: the round offset h0 only
// multiplies mode q by e^{-+2 pi i kx(q) h0 / H}, which is applied to the
// per-round partial sums (forward) or to the spectra (inverse) on the VALU.
// So a workgroup holds 64-row stages of x or y, rounds of R or Z, and its
// twiddle fragments in registers. Both kernels are persistent (one
// workgroup per resident slot, planes strided by the grid), so the rows of
// the next rounds or plane are in flight while the current one is
// multiplied; the forward keeps three rounds in a register ring.
//
// Precision. fp16 x is exact as an MFMA operand; bf16 and fp32 x are scaled
// by one power of two per 64-row round into fp16 range (fp32 as an fp16 hi
// part and an fp16 remainder), which keeps every element within 2^28 of the
// round's largest exact (bf16) or to about 22 bits (fp32); smaller ones add
// negligibly to any output. R, Z and the spectra are rounded to fp16 (fp32
// planes: hi + lo) after a power-of-two scale derived from a bound (the
// round's largest |x| times W, or the plane's largest |Y| times 4 m1), which
// keeps every fp16 operand below 2^15 and far above the subnormal range;
// every scale is undone in fp32. Twiddles are rounded to fp16 (fp32 planes:
// hi + lo).
//
// One fragment of v_mfma_f32_16x16x32 (A: 16 x 32, B: 32 x 16): lane l holds
// row / column l % 16 and the eight consecutive k = 8 (l / 16) .. +7;
// accumulator register j of lane l holds row 4 (l / 16) + j, column l % 16.

#pragma once

#include "common.hpp"

namespace fno {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

constexpr int kRows = 64;  // rows per round
constexpr int kMaxH = 256; // largest plane height

// LDS row pitches. Measured on gfx950 (bank-conflict counter over single
// access patterns): a 16-byte fragment read (lane l: row l % 16, unit l / 16)
// is conflict-free when the row pitch is 2 mod 4 sixteen-byte units and takes
// two or more passes for odd pitches or multiples of 4; a 32-bit store whose
// 16-lane row blocks are 2 rows apart is conflict-free when 2 rows are 16 mod
// 32 words. 4-byte stores go 32 lanes to a pass over 32 banks, 8-byte stores
// 16 lanes, 16-byte stores 8 lanes.
constexpr int kRBP = 144;  // halves per row of the forward R buffer (128 + pad): 18 units, 2 rows = 144 words

__device__ __forceinline__ v4f mma(u32x4 a, u32x4 b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c, 0, 0, 0);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// two fp32 -> packed fp16 pair, round to nearest even (one v_cvt_pk_f16_f32)
__device__ __forceinline__ uint32_t h16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// running maximum of the magnitude fields (sign cleared) of eight packed
// 16-bit floats, two lanes at a time (v_pk_max_u16); for finite fp16 and
// bf16 values the unsigned order of these bits is the order of magnitudes
__device__ __forceinline__ u16x2 absmax_acc(u16x2 m, u32x4 v) {
#pragma unroll
  for (int i = 0; i < 4; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, v[i] & 0x7fff7fffu));
  return m;
}

// maximum over the 16 lanes of each DPP row, in every lane of the row:
// exchanges with lane ^ 1, lane ^ 2 (quad permutes), then the mirrored lane
// of the half row and of the row (every source lane exists, so the bound
// control that zeroes missing ones never applies; it lets each move fold
// into its v_max as one DPP instruction)
__device__ __forceinline__ int row16_max(int v) {
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0xb1, 0xf, 0xf, true));   // quad_perm [1, 0, 3, 2]
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0x4e, 0xf, 0xf, true));   // quad_perm [2, 3, 0, 1]
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0x141, 0xf, 0xf, true));  // row_half_mirror
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0x140, 0xf, 0xf, true));  // row_mirror
  return v;
}

// maximum over the wave, uniform: rows reduced by DPP, the four row results
// read into scalars
__device__ __forceinline__ int wave_max_i32(int v) {
  v = row16_max(v);
  const int a = max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16));
  const int b = max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48));
  return max(a, b);
}

// maximum of non-negative floats over the wave (their bit patterns order
// the same way as signed integers)
__device__ __forceinline__ float wave_max_f32(float v) {
  return __int_as_float(wave_max_i32(__float_as_int(v)));
}

// ------------------------------------------------------------------ forward

constexpr int kFT = 256;  // threads per workgroup of the inverse plane kernel (4 waves)

// Storage policy: fp32 planes are carried as fp16 hi + lo parts (two
// operands, three products per pair, hi*hi + hi*lo + lo*hi); fp16 and bf16
// planes as one fp16 part.
template <int DT>
struct MxPol {
  static constexpr bool SP = DT == DT_F32;  // split operands
  static constexpr int NP = SP ? 2 : 1;     // fp16 parts per operand
  static constexpr int ES = SP ? 4 : 2;     // storage bytes per element
};

// Accumulator chains: a dependent MFMA waits for its predecessor's result,
// so products are spread over independent accumulators (hi*hi and the two
// cross terms apart; with KS, even and odd K blocks apart) and summed at the
// end.
template <bool KS>
struct AccN {
  v4f c[2][KS ? 2 : 1];  // [cross terms][odd block]
  __device__ __forceinline__ AccN() {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < (KS ? 2 : 1); ++j) c[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  __device__ __forceinline__ void add(const u32x4 (&a)[2], const u32x4 (&b)[2], int kb, bool sp) {
    const int j = KS ? (kb & 1) : 0;
    c[0][j] = mma(a[0], b[0], c[0][j]);
    if (sp) {
      c[1][j] = mma(a[0], b[1], c[1][j]);
      c[1][j] = mma(a[1], b[0], c[1][j]);
    }
  }
  __device__ __forceinline__ v4f sum(bool sp) const {
    v4f r = c[0][0];
    if (KS) r += c[0][KS ? 1 : 0];
    if (sp) {
      r += c[1][0];
      if (KS) r += c[1][KS ? 1 : 0];
    }
    return r;
  }
};

// fp32 -> fp16 hi, fp16 lo = fp16(v - hi), packed for two values
__device__ __forceinline__ void split2(float v0, float v1, uint32_t &hi, uint32_t &lo) {
  const f32x2 v = {v0, v1};
  const f16x2 h = __builtin_convertvector(v, f16x2);
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(v - __builtin_convertvector(h, f32x2), f16x2));
}

constexpr int kPF = 3;  // rounds in flight per workgroup (register ring)

// lgr: log2 rounds per plane; total: rounds of this workgroup; bid / nblk:
// this workgroup's index among the nblk workgroups sharing the planes
struct FwdShape {
  int H, m1, m2, NT, MT, NN, lgW, lgr, total, bid, nblk;
};

// rows of global round g of this workgroup: plane bid + (g >> lgr) * nblk,
// rows 64 (g mod 2^lgr) .. +63; FU 16-byte units per thread of a workgroup
// of NW waves
template <int DT, int KB, int NW>
struct FwdIO {
  static constexpr int NT = NW * 64;                               // threads
  static constexpr int W = 32 * KB, UR = W * MxPol<DT>::ES / 16;  // 16-byte units per row
  static constexpr int FU = kRows * UR / NT;                       // units per thread and round
};

// TW: two plane sets in one launch (planes past nsplit from x2); compiled
// separately so that the one-set kernels carry no selection
template <int DT, int KB, int NW, bool TW>
__device__ __forceinline__ void fwd_fetch(const PlaneMxFwdArgs &a, int g, const FwdShape &s, int tid,
                                          u32x4 (&p)[FwdIO<DT, KB, NW>::FU]) {
  using IO = FwdIO<DT, KB, NW>;
  const int lgr = s.lgr, H = s.H;
  size_t plane = (size_t)s.bid + (size_t)(g >> lgr) * s.nblk;
  const void *x = a.x;
  if constexpr (TW) {
    if (plane >= (size_t)a.nsplit) {  // the second plane set (uniform per workgroup)
      x = a.x2;
      plane -= a.nsplit;
    }
  }
  const int r = g & ((1 << lgr) - 1);
  const u32x4 *src = reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(x) + plane * H * IO::W * MxPol<DT>::ES) +
                     (size_t)r * kRows * IO::UR + tid;
  // x is read once: non-temporal loads keep it from displacing the
  // spectra and tables the next kernels read from the caches
#pragma unroll
  for (int v = 0; v < IO::FU; ++v) p[v] = __builtin_nontemporal_load(src + v * IO::NT);
}

// eight bf16 -> eight fp16 times 2^sig (exact while the result is normal)
__device__ __forceinline__ u32x4 bf16_to_f16_scaled(u32x4 d, float sc) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(d[i] << 16) * sc, hi = __uint_as_float(d[i] & 0xffff0000u) * sc;
    o[i] = h16x2(lo, hi);
  }
  return o;
}

template <int DT, int KB, int CPW>
struct FwdRegs {
  static constexpr int NP = MxPol<DT>::NP;
  u32x4 th[CPW][NP][KB];  // row twiddles (A operand) of this wave's c-tiles
  u32x4 ef[NP][4];                // column twiddles (A operand) of this wave's m-tile
};

// LDS of the forward kernel: two buffers of each per-round stage, so that
// one barrier per round suffices (round g writes buffer g & 1 while round
// g - 1's buffer is still being read)
template <int DT, int KB>
struct FwdLds {
  static constexpr int NP = MxPol<DT>::NP;
  static constexpr int PITCH = 4 * KB + 2;       // staged row: W halves + pad, in 16-byte units (2 mod 4)
  static constexpr int STG = kRows * PITCH;      // units per stage part
  static constexpr int RBS = 32 * kRBP;          // halves per R part
  u32x4 *stage;   // [2][NP][64][PITCH]
  uint16_t *rb;   // [2][NP][32][kRBP]
  float2 *twh;    // [H]
  int *mxs;       // [2][8] per-wave largest exponents of a round
  __device__ __forceinline__ FwdLds(u32x4 *lds, int H) {
    stage = lds;
    rb = reinterpret_cast<uint16_t *>(stage + 2 * NP * STG);
    twh = reinterpret_cast<float2 *>(rb + 2 * NP * RBS);
    mxs = reinterpret_cast<int *>(twh + H);
  }
};

// largest exponent e of a round's magnitudes (all < 2^e), from the running
// maximum of one thread's share: fp16 / bf16 magnitude bits, or fp32 bits
template <int DT>
__device__ __forceinline__ int fwd_exp(uint32_t m) {
  if (!m) return -1000;
  if constexpr (DT == DT_F32) return (int)max(m >> 23, 1u) - 126;
  else if constexpr (DT == DT_BF16) return (int)max(m >> 7, 1u) - 126;
  else return (int)max(m >> 10, 1u) - 14;
}

template <int DT, int FU>
__device__ __forceinline__ uint32_t fwd_absmax(const u32x4 (&p)[FU]) {
  if constexpr (DT == DT_F32) {
    float m = 0.f;
#pragma unroll
    for (int v = 0; v < FU; ++v) m = fmaxf(fmaxf(m, fmaxf(fabsf(__uint_as_float(p[v][0])), fabsf(__uint_as_float(p[v][1])))),
                                          fmaxf(fabsf(__uint_as_float(p[v][2])), fabsf(__uint_as_float(p[v][3]))));
    return __float_as_uint(m);
  } else {
    u16x2 m = {0, 0};
#pragma unroll
    for (int v = 0; v < FU; ++v) m = absmax_acc(m, p[v]);
    return max((uint32_t)m.x, (uint32_t)m.y);
  }
}

// record this wave's largest exponent of the round whose rows are in p
template <int DT, int KB, int NW>
__device__ __forceinline__ void fwd_note(int g, const u32x4 (&p)[FwdIO<DT, KB, NW>::FU], const FwdLds<DT, KB> &L) {
  const int e = fwd_exp<DT>((uint32_t)wave_max_i32((int)fwd_absmax<DT, FwdIO<DT, KB, NW>::FU>(p)));
  if ((threadIdx.x & 63) == 0) L.mxs[(g & 1) * 8 + (threadIdx.x >> 6)] = e;
}

// largest exponent of round g over the workgroup's waves
template <int DT, int KB, int NW>
__device__ __forceinline__ int fwd_round_exp(int g, const FwdLds<DT, KB> &L) {
  int er = -1000;
#pragma unroll
  for (int i = 0; i < NW; ++i) er = max(er, L.mxs[(g & 1) * 8 + i]);
  return er;
}

// 1. stage the rows of round g (registers p) in LDS buffer g & 1 as fp16,
//    then reuse p for round g + kPF. fp16 rows go as they are, and their
//    largest exponent is noted for the R scale. bf16 and fp32 rows are
//    scaled by 2^sig into fp16 range (fp32 as hi + lo parts), with sig from
//    the round's largest exponent, noted one step earlier; this step notes
//    that of round g + 1 (registers pn). Returns sig; er: round g's largest
//    exponent for bf16 / fp32 (read here, before the slot is refilled by the
//    next step), -1000 for fp16 (read after the barrier instead).
template <int DT, int KB, int NW, bool TW>
__device__ __forceinline__ int fwd_put(int g, const FwdShape &s, u32x4 (&p)[FwdIO<DT, KB, NW>::FU],
                                       const u32x4 (&pn)[FwdIO<DT, KB, NW>::FU], const PlaneMxFwdArgs &a,
                                       const FwdLds<DT, KB> &L, int &er_out) {
  using P = MxPol<DT>;
  constexpr bool BF = DT == DT_BF16, SP = P::SP;
  constexpr int PITCH = FwdLds<DT, KB>::PITCH, STG = FwdLds<DT, KB>::STG;
  constexpr int UR = FwdIO<DT, KB, NW>::UR, FU = FwdIO<DT, KB, NW>::FU, NT = FwdIO<DT, KB, NW>::NT;
  const int tid = threadIdx.x;
  u32x4 *stage = L.stage + (g & 1) * P::NP * STG;
  int sig = 0;
  er_out = -1000;
  if constexpr (BF || SP) {
    const int er = fwd_round_exp<DT, KB, NW>(g, L);
    sig = er > -1000 ? max(-120, min(120, 14 - er)) : 0;  // round max * 2^sig < 2^15
    er_out = er;
  }
  const float sc = pow2f(sig);
#pragma unroll
  for (int v = 0; v < FU; ++v) {
    const int e = v * NT + tid;
    const int row = e / UR, cu = e - row * UR;
    const u32x4 d = p[v];
    if constexpr (SP) {
      uint32_t h0, l0, h1, l1;
      split2(__uint_as_float(d[0]) * sc, __uint_as_float(d[1]) * sc, h0, l0);
      split2(__uint_as_float(d[2]) * sc, __uint_as_float(d[3]) * sc, h1, l1);
      reinterpret_cast<uint2 *>(stage + row * PITCH)[cu] = make_uint2(h0, h1);
      reinterpret_cast<uint2 *>(stage + STG + row * PITCH)[cu] = make_uint2(l0, l1);
    } else if constexpr (BF) {
      stage[row * PITCH + cu] = bf16_to_f16_scaled(d, sc);
    } else {
      stage[row * PITCH + cu] = d;
    }
  }
  if constexpr (BF || SP) fwd_note<DT, KB, NW>(g + 1, pn, L);
  else fwd_note<DT, KB, NW>(g, p, L);
  // unconditional, so that the compiler counts loads exactly; past the end
  // it re-reads the last round (an L2 hit), never used
  fwd_fetch<DT, KB, NW, TW>(a, min(g + kPF, s.total - 1), s, tid, p);
  return sig;
}

// round g's R scale exponent: |R| <= W max|x| < 2^(e + lgW), so R 2^se <
// 2^15; for staged bf16 / fp32 rows (max < 2^15) that is -lgW
template <int DT, int KB, int NW>
__device__ __forceinline__ int fwd_scale(int g, const FwdShape &s, const FwdLds<DT, KB> &L) {
  if constexpr (DT == DT_BF16 || DT == DT_F32) return -s.lgW;
  const int er = fwd_round_exp<DT, KB, NW>(g, L);
  return er > -1000 ? max(-120, min(120, 15 - er - s.lgW)) : 0;
}

// 2. row product of round g, transposed: R^T[c][h] = sum_w T[w][c] x[h][w]
//    with the twiddles as the register-held A operand (CPW 16-column tiles
//    of R per wave) and the staged rows as B; R scaled by 2^se (undone in
//    fwd_col) into fp16 pairs of LDS buffer g & 1. The jobs (16-row block,
//    group of CPW c-tiles) are dealt to the NW waves round-robin; NW is a
//    multiple of the groups per block, so a wave's c-tiles never change.
template <int DT, int KB, int CPW, int NW>
__device__ __forceinline__ void fwd_row(int g, int se, const FwdShape &s, const FwdLds<DT, KB> &L,
                                        const FwdRegs<DT, KB, CPW> &R) {
  constexpr bool TWO = CPW == 2;
  using P = MxPol<DT>;
  constexpr bool BF = DT == DT_BF16, SP = P::SP;
  constexpr int NP = P::NP;
  constexpr int PITCH = FwdLds<DT, KB>::PITCH, STG = FwdLds<DT, KB>::STG, RBS = FwdLds<DT, KB>::RBS;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const u32x4 *stage = L.stage + (g & 1) * NP * STG;
  uint16_t *rb = L.rb + (g & 1) * NP * RBS;
  const int G = s.NT / CPW;  // c-tile groups per 16-row block
  const int ct0 = (wv % G) * CPW;
  // fragments are read in groups of KG blocks ahead of their products
  constexpr int KG = SP && KB > 2 ? 2 : KB;
  for (int st = wv / G; st < 4; st += NW / G) {
    const u32x4 *br = stage + (st * 16 + (lane & 15)) * PITCH + (lane >> 4);
    AccN<!TWO> a0, a1;  // two tiles already give independent chains
#pragma unroll
    for (int k0 = 0; k0 < KB; k0 += KG) {
      u32x4 bv[KG][2];
#pragma unroll
      for (int kb = 0; kb < KG; ++kb)
#pragma unroll
        for (int q = 0; q < 2; ++q) bv[kb][q] = q < NP ? br[q * STG + (k0 + kb) * 4] : bv[kb][0];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kb = 0; kb < KG; ++kb) {
        const u32x4 t0[2] = {R.th[0][0][k0 + kb], R.th[0][NP - 1][k0 + kb]};
        a0.add(t0, bv[kb], kb, SP);
        if constexpr (TWO) {
          const u32x4 t1[2] = {R.th[1][0][k0 + kb], R.th[1][NP - 1][k0 + kb]};
          a1.add(t1, bv[kb], kb, SP);
        }
      }
    }
    const v4f acc0 = a0.sum(SP), acc1 = TWO ? a1.sum(SP) : acc0;
    const int h = st * 16 + (lane & 15);
    const float f = pow2f(se);
    uint32_t *col = reinterpret_cast<uint32_t *>(rb) + h;
#pragma unroll
    for (int t = 0; t < (TWO ? 2 : 1); ++t) {
      const v4f &acc = t == 0 ? acc0 : acc1;
      const int ky0 = 8 * (ct0 + t) + 2 * (lane >> 4);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (ky0 + j < s.m2) {
          uint32_t hi, lo;
          split2(acc[2 * j] * f, acc[2 * j + 1] * f, hi, lo);
          col[(ky0 + j) * (kRBP / 2)] = hi;
          if constexpr (SP) col[RBS / 2 + (ky0 + j) * (kRBP / 2)] = lo;
        }
      }
    }
  }
}

// 3. column product of round g's R against the 64-row twiddle block (m-tile
//    wv of the modes), phase-shifted by the round offset and unscaled into X;
//    after the last round of a plane, X is scaled, stored and reset. pe: the
//    plane's largest input exponent (every |x| < 2^pe, so every |X| < 2^pe
//    after the 1 / (H W) scale), which sets the power-of-two scale of the
//    half exchange: |X| 2^(14 - pe) < 2^14, and every value down to 2^-28 of
//    the plane's largest input stays a normal fp16.
template <int DT, int KB, int CPW, bool TW>
__device__ __forceinline__ void fwd_col(int g, int se, int pe, const FwdShape &s, const PlaneMxFwdArgs &a,
                                        const FwdLds<DT, KB> &L, const FwdRegs<DT, KB, CPW> &R, float2 (&X)[2][2]) {
  using P = MxPol<DT>;
  constexpr bool SP = P::SP;
  constexpr int NP = P::NP;
  constexpr int RBS = FwdLds<DT, KB>::RBS;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (wv >= s.MT) return;
  const int r = g & ((1 << s.lgr) - 1);
  const uint16_t *rb = L.rb + (g & 1) * NP * RBS;
  const float isc = pow2f(-se);
  float2 ph[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int q = 8 * wv + 2 * (lane >> 4) + t;
    const int kx = q < s.m1 ? q : s.H - 2 * s.m1 + q;
    ph[t] = L.twh[(kx * kRows * r) & (s.H - 1)];
  }
  // fragments of NB ky tiles at a time (both for fp16 parts, one for
  // hi + lo parts), then their products as independent chains
  constexpr int NB = SP ? 1 : 2;
#pragma unroll
  for (int n0 = 0; n0 < 2; n0 += NB) {
    if (n0 < s.NN) {
      u32x4 bv[NB][4][2];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int nn = n0 + i < s.NN ? n0 + i : n0;
        const u32x4 *br = reinterpret_cast<const u32x4 *>(rb + (nn * 16 + (lane & 15)) * kRBP) + (lane >> 4);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int q = 0; q < 2; ++q) bv[i][kb][q] = q < NP ? br[q * (RBS / 8) + kb * 4] : bv[i][kb][0];
      }
      __builtin_amdgcn_sched_barrier(0);
      AccN<SP> ac[NB];  // two ky tiles give independent chains unless split
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const u32x4 e2[2] = {R.ef[0][kb], R.ef[NP - 1][kb]};
#pragma unroll
        for (int i = 0; i < NB; ++i)
          if (n0 + i < s.NN) ac[i].add(e2, bv[i][kb], kb, SP);
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        if (n0 + i < s.NN) {
          const v4f acc = ac[i].sum(SP);
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const float yr = acc[2 * t] * isc, yi = acc[2 * t + 1] * isc;
            X[n0 + i][t].x += yr * ph[t].x - yi * ph[t].y;
            X[n0 + i][t].y += yr * ph[t].y + yi * ph[t].x;
          }
        }
      }
    }
  }
  if (r == (1 << s.lgr) - 1) {
    const size_t plane = (size_t)s.bid + (size_t)(g >> s.lgr) * s.nblk;
    uint32_t *o16 = a.out16;
    int *oe = a.oexp;
    size_t lp = plane;  // index within its plane set
    if constexpr (TW) {
      if (plane >= (size_t)a.nsplit) {
        o16 = a.out16_2;
        oe = a.oexp2;
        lp = plane - a.nsplit;
      }
    }
    if (o16) {
      const int sx = pe > -1000 ? max(-120, min(120, 14 - pe)) : 0;
      const float f = a.scale * pow2f(sx);
      uint32_t *op = o16 + lp * (2 * s.m1 * s.m2);
#pragma unroll
      for (int nn = 0; nn < 2; ++nn) {
        const int ky = nn * 16 + (lane & 15);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int q = 8 * wv + 2 * (lane >> 4) + t;
          if (nn < s.NN && ky < s.m2 && q < 2 * s.m1) op[q * s.m2 + ky] = h16x2(X[nn][t].x * f, X[nn][t].y * f);
          X[nn][t] = make_float2(0.f, 0.f);
        }
      }
      if (threadIdx.x == 0) oe[lp] = sx;
      return;
    }
    float2 *op = a.out + plane * (2 * s.m1 * s.m2);
    if constexpr (TW) {
      if (plane >= (size_t)a.nsplit) op = a.out2 + (plane - a.nsplit) * (2 * s.m1 * s.m2);
    }
#pragma unroll
    for (int nn = 0; nn < 2; ++nn) {
      const int ky = nn * 16 + (lane & 15);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int q = 8 * wv + 2 * (lane >> 4) + t;
        if (nn < s.NN && ky < s.m2 && q < 2 * s.m1)
          op[q * s.m2 + ky] = make_float2(X[nn][t].x * a.scale, X[nn][t].y * a.scale);
        X[nn][t] = make_float2(0.f, 0.f);
      }
    }
  }
}

// One pipeline step: stage round g, one barrier, then round g's row product
// and round g - 1's column product (different LDS buffers).
// se_prev: total scale exponent of round g - 1's R (staging and R scale);
// pe: largest input exponent of the rounds so far of round g - 1's plane
// (then of round g's)
template <int DT, int KB, int CPW, int NW, bool TW>
__device__ __forceinline__ void fwd_step(int g, int &se_prev, int &pe, const FwdShape &s,
                                         u32x4 (&p)[FwdIO<DT, KB, NW>::FU], const u32x4 (&pn)[FwdIO<DT, KB, NW>::FU],
                                         const PlaneMxFwdArgs &a, const FwdLds<DT, KB> &L,
                                         const FwdRegs<DT, KB, CPW> &R, float2 (&X)[2][2]) {
  int eg;
  const int sig = fwd_put<DT, KB, NW, TW>(g, s, p, pn, a, L, eg);
  __syncthreads();
  const int se = fwd_scale<DT, KB, NW>(g, s, L);
  // fp16: round g's exponents were noted in this step's staging; their slot
  // is refilled two steps later, after the next barrier
  if constexpr (DT == DT_F16) eg = fwd_round_exp<DT, KB, NW>(g, L);
  fwd_row<DT, KB, CPW, NW>(g, se, s, L, R);
  if (g > 0) fwd_col<DT, KB, CPW, TW>(g - 1, se_prev, pe, s, a, L, R, X);
  se_prev = se + sig;
  pe = (g & ((1 << s.lgr) - 1)) == 0 ? eg : max(pe, eg);
}

// Persistent: workgroup b of nblk transforms planes b, b + nblk, ...; its rounds
// form one stream with kPF rounds in flight in a register ring, across plane
// boundaries. NW waves per workgroup: 8 (one workgroup per CU) for wide or
// split-operand planes and more than four m-tiles, else 4 (two or more per
// CU). CPW: R c-tiles per wave in the row product (2 only when that still
// gives every wave a job).
// Workgroup bid of nblk (NW waves): planes bid, bid + nblk, ...; LDS at lds.
template <int DT, int KB, int CPW, int NW, bool TW>
__device__ __forceinline__ void fwd_mx_run(const PlaneMxFwdArgs &a, int bid, int nblk, u32x4 *lds) {
  using P = MxPol<DT>;
  using IO = FwdIO<DT, KB, NW>;
  constexpr int NP = P::NP;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int lgr = a.H == 256 ? 2 : a.H == 128 ? 1 : 0;
  const int nmine = (a.nplanes - bid + nblk - 1) / nblk;
  const FwdShape s{a.H, a.m1, a.m2, a.nt, a.mt, a.nn, a.lgW, lgr, nmine << lgr, bid, nblk};
  const FwdLds<DT, KB> L(lds, s.H);
  if (s.total < 1) return;

  // Round 0's rows are requested first and the twiddle tables next (L2
  // hits), so that the two latencies overlap; both are waited for, then
  // rounds 1 and 2 go out in ring order. Every fetch is unconditional
  // (clamped to the last round) and the loop below runs whole ring turns
  // only, with the remainder after it: a path that left the loop early but
  // reached its head would make the compiler wait for all loads in flight
  // there, draining the ring every turn.
  u32x4 p0[IO::FU], p1[IO::FU], p2[IO::FU];
  fwd_fetch<DT, KB, NW, TW>(a, 0, s, tid, p0);
  __builtin_amdgcn_sched_barrier(0);

  FwdRegs<DT, KB, CPW> R;
  const int G = s.NT / CPW;
#pragma unroll
  for (int t = 0; t < CPW; ++t) {
    const int ct = min((wv % G) * CPW + t, s.NT - 1);
#pragma unroll
    for (int q = 0; q < NP; ++q)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        R.th[t][q][kb] = reinterpret_cast<const u32x4 *>(q ? a.tf_lo : a.tf)[((size_t)ct * KB + kb) * 64 + lane];
  }
  {
    const int mt = min(wv, s.MT - 1);
#pragma unroll
    for (int q = 0; q < NP; ++q)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        R.ef[q][kb] = reinterpret_cast<const u32x4 *>(q ? a.ef_lo : a.ef)[((size_t)mt * 4 + kb) * 64 + lane];
  }

  float2 tw[(kMaxH + IO::NT - 1) / IO::NT];
#pragma unroll
  for (int i = 0; i < (kMaxH + IO::NT - 1) / IO::NT; ++i) {
    const int v = tid + i * IO::NT;
    if (v < s.H) tw[i] = a.tw_h[v];
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  __builtin_amdgcn_sched_barrier(0);
  fwd_fetch<DT, KB, NW, TW>(a, min(1, s.total - 1), s, tid, p1);
  __builtin_amdgcn_sched_barrier(0);
  fwd_fetch<DT, KB, NW, TW>(a, min(2, s.total - 1), s, tid, p2);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < (kMaxH + IO::NT - 1) / IO::NT; ++i) {
    const int v = tid + i * IO::NT;
    if (v < s.H) L.twh[v] = tw[i];
  }
  float2 X[2][2];
#pragma unroll
  for (int nn = 0; nn < 2; ++nn)
#pragma unroll
    for (int t = 0; t < 2; ++t) X[nn][t] = make_float2(0.f, 0.f);
  // scaled dtypes: round 0's largest exponent before its staging
  if constexpr (P::SP || DT == DT_BF16) {
    fwd_note<DT, KB, NW>(0, p0, L);
    __syncthreads();
  }
  int se_prev = 0, pe = -1000;
  const int full = s.total - s.total % kPF;
  int g = 0;
  for (; g < full; g += kPF) {
    fwd_step<DT, KB, CPW, NW, TW>(g, se_prev, pe, s, p0, p1, a, L, R, X);
    fwd_step<DT, KB, CPW, NW, TW>(g + 1, se_prev, pe, s, p1, p2, a, L, R, X);
    fwd_step<DT, KB, CPW, NW, TW>(g + 2, se_prev, pe, s, p2, p0, a, L, R, X);
  }
  if (g < s.total) fwd_step<DT, KB, CPW, NW, TW>(g, se_prev, pe, s, p0, p1, a, L, R, X);
  if (g + 1 < s.total) fwd_step<DT, KB, CPW, NW, TW>(g + 1, se_prev, pe, s, p1, p2, a, L, R, X);
  __syncthreads();
  fwd_col<DT, KB, CPW, TW>(s.total - 1, se_prev, pe, s, a, L, R, X);
}

// ------------------------------------------------------------------ inverse

// Inverse sizes: up to 32 kx per corner and 32 ky, or (SM) up to 16 of each.
// The spectra buffer holds YR ky rows of 2 (2 m1) halves plus 16 of padding
// (pitch 18 or 10 units), Z 64 rows of 2 m2 halves plus 16 (pitch 10 or 6
// units, and 2 rows apart 80 or 48 words): the fragment reads and the Z
// stores are conflict-free.
template <bool SM>
struct InvGeom {
  static constexpr int NY = SM ? 2 : 8;         // spectra values per thread (K <= 512 or 2048)
  static constexpr int KBM = SM ? 2 : 4;        // k-blocks of E' Y
  static constexpr int NNM = SM ? 1 : 2;        // ky tiles
  static constexpr int YR = SM ? 16 : 32;       // ky rows of the spectra buffer
  static constexpr int YP = SM ? 80 : 144;      // halves per spectra row
  static constexpr int ZP = SM ? 48 : 80;       // halves per Z row
};

// The spectra of a plane are dealt to the 256 threads in tiles of 8 kx rows
// (q) by 4 ky, ky tiles fastest (2^lgk of them: ceil(m2 / 4) rounded up to a
// power of two): value i of thread t is in tile t / 32 + 8 i, at row
// (t / 4) % 8 and ky t % 4 of it. So the 32 lanes of one store into the
// [ky][q] spectra buffer cover 8 consecutive q of 4 rows, on 32 distinct
// banks (with the whole plane in one thread-column, 32 lanes wrote one q of
// 32 rows: four or eight to a bank), and a global load still reads runs of
// consecutive modes. 8 NY tiles hold every mode: 2 m1 / 8 <= 8 (4 for SM)
// row tiles of at most 8 (4) ky tiles.
struct InvMap {
  int m1, m2, lgk;
};

// mode index (q m2 + ky) of value i of thread tid, or -1 for tile padding
__device__ __forceinline__ int inv_mode(const InvMap &mp, int i, int tid, int &q, int &ky) {
  const int tile = (tid >> 5) + 8 * i;
  q = 8 * (tile >> mp.lgk) + ((tid >> 2) & 7);
  ky = 4 * (tile & ((1 << mp.lgk) - 1)) + (tid & 3);
  return q < 2 * mp.m1 && ky < mp.m2 ? q * mp.m2 + ky : -1;
}

// spectra of one plane into registers (zero for tile padding)
template <int NY>
__device__ __forceinline__ void inv_load(const float2 *in, size_t plane, const InvMap &mp, int tid, float2 (&yv)[NY]) {
  const float2 *ip = in + plane * (size_t)(2 * mp.m1 * mp.m2);
#pragma unroll
  for (int i = 0; i < NY; ++i) {
    int q, ky;
    const int k = inv_mode(mp, i, tid, q, ky);
    const float2 t = ip[max(k, 0)];
    yv[i] = k >= 0 ? t : make_float2(0.f, 0.f);
  }
}

// the same from the half exchange: fp16 pairs and the exponent of each group
// of four modes, kept raw (decoded by inv_decode once they are needed, so the
// loads stay in flight)
template <int NY>
__device__ __forceinline__ void inv_load16(const uint32_t *in, const signed char *ex, size_t plane, const InvMap &mp,
                                           int tid, uint32_t (&hv)[NY], int (&ev)[NY]) {
  const int K = 2 * mp.m1 * mp.m2;
  const uint32_t *ip = in + plane * K;
  const signed char *ep = ex + plane * ((K + 3) >> 2);
#pragma unroll
  for (int i = 0; i < NY; ++i) {
    int q, ky;
    const int k = max(inv_mode(mp, i, tid, q, ky), 0);
    hv[i] = ip[k];
    ev[i] = ep[k >> 2];
  }
}

template <int NY>
__device__ __forceinline__ void inv_decode(const InvMap &mp, int tid, const uint32_t (&hv)[NY], const int (&ev)[NY],
                                           float2 (&yv)[NY]) {
#pragma unroll
  for (int i = 0; i < NY; ++i) {
    // each half converted on its own (as in the contraction's weight split)
    const float sc = pow2f(-ev[i]);
    const float re = (float)__builtin_bit_cast(_Float16, (uint16_t)(hv[i] & 0xffffu)) * sc;
    const float im = (float)__builtin_bit_cast(_Float16, (uint16_t)(hv[i] >> 16)) * sc;
    int q, ky;
    yv[i] = inv_mode(mp, i, tid, q, ky) >= 0 ? make_float2(re, im) : make_float2(0.f, 0.f);
  }
}

// Persistent: workgroup b of nblk transforms planes b, b + nblk, ...; the
// spectra of the next plane are requested before the current plane's last
// round. Per round of 64 output rows:
//  1. phase-rotate the spectra by the round offset, scale, fp16 into LDS;
//  2. Z = E' Y (two m-tiles of rows per wave), fp16 into LDS;
//  3. y^T[w][h] = sum_c T'[c][w] Z[h][c] with the twiddles as the
//     register-held A operand, so each lane holds four consecutive outputs
//     of a row; unscaled, rounded to the storage dtype into the out stage;
//  4. coalesced 16-byte stores of the 64 rows.
// fp32 planes carry the spectra, Z and the twiddles as fp16 hi + lo.
// SM: at most 16 kx per corner and 16 ky, so the spectra, Z and the
// fragment registers take their smaller sizes (fewer registers and LDS,
// more workgroups per CU). HX: the spectra come as the half exchange (fp16
// pairs with exponents), compiled separately so that each form keeps only
// its own registers. ZOUT (fp16 / bf16 only): steps 3 and 4 are replaced by
// a copy of the round's Z rows (scaled fp16 pairs) to a.zg, for a consumer
// that applies the row stage itself.
template <int DT, int KB, bool SM, bool HX = false, bool ZOUT = false>
__device__ __forceinline__ void inv_mx_run(const PlaneMxInvArgs &a, int bid, int nblk, u32x4 *lds) {
  using P = MxPol<DT>;
  using G = InvGeom<SM>;
  constexpr bool SP = P::SP;
  constexpr int NP = P::NP;
  constexpr int W = 32 * KB;
  constexpr int UR = W * P::ES / 16, OP = UR + 1;  // 16-byte units per output row, stage pitch
  constexpr int FU = KB * P::ES / 2;               // 16-byte output units per thread and round
  constexpr int NTW = W / 16;                      // output column tiles
  constexpr int NPW = NTW / 4;                     // column tiles per wave
  constexpr int NY = G::NY;                        // spectra values per thread
  constexpr int KBM = G::KBM, NNM = G::NNM;        // most k-blocks of E' Y, ky tiles
  constexpr int YP = G::YP, ZP = G::ZP;            // pitches (halves) of the spectra and Z rows
  constexpr int YBS = G::YR * YP, ZBS = kRows * ZP;  // halves per part
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int H = a.H, m1 = a.m1, m2 = a.m2, NN = a.nn, KB1 = a.kb1;
  const int nk = (m2 + 3) >> 2;  // ky tiles of the spectra mapping
  const InvMap mp{m1, m2, nk <= 1 ? 0 : nk <= 2 ? 1 : nk <= 4 ? 2 : 3};
  u32x4 *ostage = lds;                                                      // [64][OP]
  uint16_t *yb = reinterpret_cast<uint16_t *>(ostage + kRows * OP);         // [NP][YR][YP]
  uint16_t *zb = yb + NP * YBS;                                             // [NP][64][ZP]
  float2 *twh = reinterpret_cast<float2 *>(zb + NP * ZBS);                  // [H]
  float *ymx = reinterpret_cast<float *>(twh + H);                          // [2][4]

  float2 yv[NY], yn[NY];
  uint32_t hn[NY];
  int en[NY];
  constexpr bool half = HX;
  int cur = bid;  // < nplanes: the grid is never larger
  if (cur < a.nplanes) {
    if constexpr (half) {
      inv_load16<NY>(a.in16, a.iexp, bid, mp, tid, hn, en);
      inv_decode<NY>(mp, tid, hn, en, yv);
    } else {
      inv_load<NY>(a.in, bid, mp, tid, yv);
    }
  }
  for (int v = tid; v < NP * YBS / 2; v += kFT) reinterpret_cast<uint32_t *>(yb)[v] = 0u;
  for (int v = tid; v < H; v += kFT) twh[v] = a.tw_h[v];

  // E' fragments of m-tiles 2 wv, 2 wv + 1 (rows j = 16 wv .. 16 wv + 15)
  u32x4 ef[2][KBM][NP];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int kb = 0; kb < KBM; ++kb)
#pragma unroll
      for (int q = 0; q < NP; ++q) {
        const u32x4 t = reinterpret_cast<const u32x4 *>(q ? a.ef_lo : a.ef)[((size_t)(2 * wv + mi) * KB1 + (kb < KB1 ? kb : 0)) * 64 + lane];
        ef[mi][kb][q] = kb < KB1 ? t : u32x4{0u, 0u, 0u, 0u};
      }
  // T' fragments (A operand) of output column tiles wv, wv + 4, ...
  u32x4 tb[NPW][NNM][NP];
#pragma unroll
  for (int i = 0; i < NPW; ++i)
#pragma unroll
    for (int kb = 0; kb < NNM; ++kb)
#pragma unroll
      for (int q = 0; q < NP; ++q) {
        if constexpr (!ZOUT) {
          const u32x4 t =
              reinterpret_cast<const u32x4 *>(q ? a.tb_lo : a.tb)[((size_t)(wv + 4 * i) * NN + (kb < NN ? kb : 0)) * 64 + lane];
          tb[i][kb][q] = kb < NN ? t : u32x4{0u, 0u, 0u, 0u};
        }
      }

  const int rounds = H / kRows;
  for (int pi = 0; cur < a.nplanes; ++pi) {
    const size_t plane = (size_t)cur;
    const int nxt = cur + nblk;
    float mloc = 0.f;
#pragma unroll
    for (int i = 0; i < NY; ++i) mloc = fmaxf(mloc, fmaxf(fabsf(yv[i].x), fabsf(yv[i].y)));
    mloc = wave_max_f32(mloc);
    if (lane == 0) ymx[(pi & 1) * 4 + wv] = mloc;
    __syncthreads();

    // |Z| <= sum_q (|Re Y| + |Im Y|) <= 4 m1 max|Y| < 2^(e + lg4m1)
    float ym = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) ym = fmaxf(ym, ymx[(pi & 1) * 4 + i]);
    int e = 0;
    if (ym > 0.f) (void)frexpf(ym, &e);
    const int se = ym > 0.f ? max(-120, min(120, 15 - e - a.lg4m1)) : 0;
    const float sc = pow2f(se), isc = pow2f(-se);
    if constexpr (ZOUT) {
      if (tid == 0) a.zexp[plane] = (signed char)se;
    }

    u32x4 *yp = reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(a.y) + plane * H * W * P::ES);
    auto round = [&](int r) {
      // 1. spectra of the round: Y[q][ky] e^{+2 pi i kx(q) h0 / H}, scaled, fp16
#pragma unroll
      for (int i = 0; i < NY; ++i) {
        int q, ky;
        if (inv_mode(mp, i, tid, q, ky) >= 0) {
          const int kx = q < m1 ? q : H - 2 * m1 + q;
          const float2 w = twh[(kx * kRows * r) & (H - 1)];  // e^{-i theta}
          const float zr = (yv[i].x * w.x + yv[i].y * w.y) * sc;
          const float zi = (yv[i].y * w.x - yv[i].x * w.y) * sc;
          uint32_t hi, lo;
          split2(zr, zi, hi, lo);
          reinterpret_cast<uint32_t *>(yb + ky * YP)[q] = hi;
          if constexpr (SP) reinterpret_cast<uint32_t *>(yb + YBS + ky * YP)[q] = lo;
        }
      }
      __syncthreads();

      // 2. Z = E' Y, rows 16 wv .. 16 wv + 15, all ky tiles; fp16 into zb
#pragma unroll
      for (int nn = 0; nn < NNM; ++nn) {
        if (nn < NN) {
          const u32x4 *br = reinterpret_cast<const u32x4 *>(yb + (nn * 16 + (lane & 15)) * YP) + (lane >> 4);
          u32x4 bv[KBM][2];
#pragma unroll
          for (int kb = 0; kb < KBM; ++kb)
#pragma unroll
            for (int q = 0; q < 2; ++q) bv[kb][q] = q < NP ? br[q * (YBS / 8) + (kb < KB1 ? kb : 0) * 4] : bv[kb][0];
          __builtin_amdgcn_sched_barrier(0);
          AccN<!SP> ac[2];
#pragma unroll
          for (int kb = 0; kb < KBM; ++kb)
            if (kb < KB1) {
#pragma unroll
              for (int mi = 0; mi < 2; ++mi) {
                const u32x4 e2[2] = {ef[mi][kb][0], ef[mi][kb][NP - 1]};
                ac[mi].add(e2, bv[kb], kb, SP);
              }
            }
#pragma unroll
          for (int mi = 0; mi < 2; ++mi) {
            const v4f acc = ac[mi].sum(SP);
            const int j0 = 8 * (2 * wv + mi) + 2 * (lane >> 4), ky = nn * 16 + (lane & 15);
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
              uint32_t hi, lo;
              split2(acc[2 * jj], acc[2 * jj + 1], hi, lo);
              reinterpret_cast<uint32_t *>(zb + (j0 + jj) * ZP)[ky] = hi;
              if constexpr (SP) reinterpret_cast<uint32_t *>(zb + ZBS + (j0 + jj) * ZP)[ky] = lo;
            }
          }
        }
      }
      __syncthreads();

      if constexpr (ZOUT) {
        // Z rows h0 .. h0 + 63 of this plane (32 NN halves each) to zg
        const size_t bb = plane / a.zco, oo = plane - bb * a.zco;
        const int UZ = 4 * NN;  // 16-byte units per row
        for (int u = tid; u < kRows * UZ; u += kFT) {
          const int row = u / UZ, c = u - row * UZ;
          const u32x4 v = *reinterpret_cast<const u32x4 *>(zb + row * ZP + 8 * c);
          *reinterpret_cast<u32x4 *>(a.zg + (((bb * H + (size_t)r * kRows + row) * a.zco + oo) * NN * 32 + 8 * c)) = v;
        }
      } else {
        // 3. y^T = T'^T Z^T: lane gets y[h][w .. w + 3], h = 16 mt + l % 16;
        // the Z fragments of MB m-tiles are read ahead of their products
        constexpr int MB = SP ? 1 : 4;
#pragma unroll
        for (int m0 = 0; m0 < 4; m0 += MB) {
          u32x4 bz[MB][NNM][2];
#pragma unroll
          for (int mi = 0; mi < MB; ++mi) {
            const u32x4 *zr = reinterpret_cast<const u32x4 *>(zb + ((m0 + mi) * 16 + (lane & 15)) * ZP) + (lane >> 4);
#pragma unroll
            for (int kb = 0; kb < NNM; ++kb)
#pragma unroll
              for (int q = 0; q < 2; ++q) bz[mi][kb][q] = q < NP ? zr[q * (ZBS / 8) + (NN > 1 ? kb : 0) * 4] : bz[mi][kb][0];
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int mi = 0; mi < MB; ++mi) {
            const int h = (m0 + mi) * 16 + (lane & 15);
            AccN<false> ac[NPW];  // NPW tiles already give independent chains
#pragma unroll
            for (int kb = 0; kb < NNM; ++kb)
              if (kb == 0 || NN > 1) {
#pragma unroll
                for (int i = 0; i < NPW; ++i) {
                  const u32x4 t2[2] = {tb[i][kb][0], tb[i][kb][NP - 1]};
                  ac[i].add(t2, bz[mi][kb], kb, SP);
                }
              }
#pragma unroll
            for (int i = 0; i < NPW; ++i) {
              const v4f acc = ac[i].sum(SP);
              const int w = (wv + 4 * i) * 16 + 4 * (lane >> 4);
              if constexpr (SP) {
                ostage[h * OP + w / 4] = u32x4{__float_as_uint(acc[0] * isc), __float_as_uint(acc[1] * isc),
                                               __float_as_uint(acc[2] * isc), __float_as_uint(acc[3] * isc)};
              } else {
                uint2 o;
                if constexpr (DT == DT_F16) {
                  o.x = h16x2(acc[0] * isc, acc[1] * isc);
                  o.y = h16x2(acc[2] * isc, acc[3] * isc);
                } else {
                  o.x = f32x2_to_bf16x2(acc[0] * isc, acc[1] * isc);
                  o.y = f32x2_to_bf16x2(acc[2] * isc, acc[3] * isc);
                }
                // 8-byte slots of rows 8..15 of each 16 swapped in pairs: the
                // 16 rows of a store then fall on distinct banks
                reinterpret_cast<uint2 *>(ostage + h * OP)[(w / 4) ^ ((h >> 3) & 1)] = o;
              }
            }
          }
        }
        __syncthreads();

        // 4. 64 rows x W elements: coalesced 16-byte stores, non-temporal (y
        // is not read again here; it should not displace cached spectra)
#pragma unroll
        for (int v = 0; v < FU; ++v) {
          const int e2 = v * kFT + tid;
          const int row = e2 / UR, cu = e2 - row * UR;
          u32x4 o = ostage[row * OP + cu];
          if constexpr (!SP) {
            if ((row >> 3) & 1) o = u32x4{o[2], o[3], o[0], o[1]};
          }
          __builtin_nontemporal_store(o, yp + (size_t)r * kRows * UR + e2);
        }
      }
    };
    for (int r = 0; r + 1 < rounds; ++r) round(r);
    // The next plane's spectra (after the last plane, this one's again,
    // unused) are requested before the last round: only that round's stores
    // are issued after them, so the copy below waits for nothing else.
    const size_t pn = nxt < a.nplanes ? (size_t)nxt : plane;
    if constexpr (half) inv_load16<NY>(a.in16, a.iexp, pn, mp, tid, hn, en);
    else inv_load<NY>(a.in, pn, mp, tid, yn);
    round(rounds - 1);
    if constexpr (half) inv_decode<NY>(mp, tid, hn, en, yn);
#pragma unroll
    for (int i = 0; i < NY; ++i) yv[i] = yn[i];
    cur = nxt;
  }
}

}  // namespace fno
