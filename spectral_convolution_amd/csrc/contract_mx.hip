// contract_mx.hip - the per-mode complex channel contraction for fp16 / bf16
// storage on bf16 matrix cores.
//
// For every retained mode k: Yh[k] (B x Co) = Xh[k] (B x Ci) * W[k] (Ci x Co),
// complex, no conjugation, fp32 accumulation (TurboFNO write-up, sections
// 2.2 and 3.2: the per-mode weight einsum, run on matrix cores). In real form
// each mode is one product with K = (i, re/im) and N = (o, re/im):
//   A[b][(i,0)] = Re X, A[b][(i,1)] = Im X,
//   B[(i,0)][(o,0)] = Re W, B[(i,1)][(o,0)] = -Im W,
//   B[(i,0)][(o,1)] = Im W, B[(i,1)][(o,1)] = Re W.
//
// Operands are split into bf16 parts so that the products are exact to fp32
// level: the fp32 spectra as hi + lo (16 significant bits), fp16 weights as
// hi + lo (exact: 11 bits), bf16 weights as they are. Products: Xh Wh + Xl Wh
// (+ Xh Wl for fp16 weights) on v_mfma_f32_16x16x32_bf16.
//
// Half exchange (HX): the spectra arrive as fp16 pairs with one power-of-two
// exponent per (b, i) plane and leave as fp16 pairs with one exponent per
// group of four modes of a (b, o) row, chosen from the group's largest
// magnitude so that every value is below 2^14 and, down to 2^-28 of that
// largest, a normal fp16. An fp16 value splits into bf16 hi + lo exactly, so
// the products stay exact; only the roundings to fp16 are added.
//
// A workgroup owns MB = 16, 8 or 4 consecutive modes x 16 or 32 batch rows x
// 32 output channels and streams the input channels in stages of 16: the
// spectra rows [b][i][MB modes] (8 MB contiguous bytes) and weight rows [mode][i][32 o]
// (128 bytes) are loaded with 16-byte accesses one stage ahead into
// registers, split and transposed into LDS as MFMA fragments, and multiplied
// there. The results leave through LDS as rows of MB modes of Yh[b][o][k].
// Four-mode workgroups (half the LDS and registers, so more of them fit on a
// CU) are used when eight-mode ones would leave resident slots empty.
//
// Adjoint from W (WT): the backward's Xh[k] = Yh[k] W[k]^H reads the layer's
// W[k][i][o] directly. With the product's contracted index c = o and output
// n = i, a stage row (mode, n) of 16 c is 64 contiguous bytes of W, which
// go to LDS as they are: 16-byte stores straight into the fragment rows; the
// conjugation is folded into the fragment forming.

#include "common.hpp"

#include <algorithm>

namespace fno {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));

// Threads per workgroup: one wave per mode (16, 8 or 4 waves; eight-mode
// workgroups measured against 4 waves of two modes each at 256^2: 26.2 ->
// 25.1 us fp16 on the half exchange, 25.1 -> 22.4 us its adjoint, 24.7 ->
// 22.9 us bf16: twice the waves per CU to hide the stage latencies, half the
// registers per lane)
template <int MB>
constexpr int cmx_threads() { return MB * 64; }
constexpr int kIC = 16;   // input channels per stage (one 32-deep block of K)
constexpr int kOT = 32;   // output channels per workgroup (four 16-column tiles of N)
constexpr int kSP = 48;   // halves per staged fragment row (32 + 16 pad: 6 units, conflict-free fragment reads)

// two fp32 -> packed fp16 pair (a in the low half), round to nearest even
__device__ __forceinline__ uint32_t f16x2_rne(float a, float b) {
  const uint32_t lo = __builtin_bit_cast(uint16_t, (_Float16)a), hi = __builtin_bit_cast(uint16_t, (_Float16)b);
  return lo | (hi << 16);
}

__device__ __forceinline__ v4f mma_bf(u32x4 a, u32x4 b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, a), __builtin_bit_cast(b8, b), c, 0, 0, 0);
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v4f mma_f16(u32x4 a, u32x4 b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// (re, im) fp32 -> packed bf16 pairs hi = (bf16(re), bf16(im)), lo = the
// rounding remainders, each rounded to nearest even
__device__ __forceinline__ void split_pair(float re, float im, uint32_t &hi, uint32_t &lo) {
  hi = f32x2_to_bf16x2(re, im);
  lo = f32x2_to_bf16x2(re - __uint_as_float(hi << 16), im - __uint_as_float(hi & 0xffff0000u));
}

// DIRECT: fp16 weights and the half exchange multiply on fp16 matrix cores
// as they are (no hi / lo parts): the spectra of one batch row are brought
// to a common power-of-two scale, the row's smallest plane exponent, so one
// product sums every input channel in one scale.
template <int DT, int MT, int MB, bool HX>
struct CmxShape {
  static constexpr bool DIRECT = HX && DT == DT_F16;
  static constexpr int NT = cmx_threads<MB>();              // threads per workgroup
  static constexpr int MW = 1;                              // modes per wave
  static constexpr int UX = MB / 2;                         // units (two modes) per spectra / result row
  static constexpr int YO = 2 * MB + 4;                     // floats per output-channel row of the result stage (+ 4 pad)
  static constexpr int YB = kOT * YO + 4;                   // floats per batch row of the result stage
  static constexpr int BT = 16 * MT;                        // batch rows per workgroup
  static constexpr int XP = DIRECT ? 1 : 2;                 // spectra parts
  static constexpr int HL = DT == DT_F16 && !DIRECT ? 2 : 1;  // weight parts
  static constexpr int XU = MB * BT * kIC * 8 / (16 * NT);   // spectra units (two modes) per thread and stage
  static constexpr int WU = MB * kIC * kOT * 4 / (16 * NT);  // 16-byte weight units per thread and stage
  static constexpr int XB = BT * kSP;                        // halves of one (mode, part) block
  static constexpr int XS = MB * XP * XB;                   // halves of the spectra stage
  static constexpr int WS = MB * HL * kOT * kSP;           // halves of the weight stage
  static constexpr int LH = XS + WS > 32 * YB ? XS + WS : 32 * YB;  // halves before the row exponents (DIRECT)
};

// Row of batch row b in the spectra block of mode m: rotated by one row per
// mode pair, so that the four mode pairs one store instruction touches
// start 24, 16 or 8 banks apart (rows of 24 words).
template <int MT>
__device__ __forceinline__ int xrow(int m, int b) { return (b + (m >> 1)) & (16 * MT - 1); }

// Row of output channel o in a mode's weight block: the two low bits of o
// and the next two swap places, so that the four output groups (4 c + t for
// c = 0 .. 3) one store instruction touches land 24 words apart mod 32
// (rows of 24 words, 4 rows apart would share banks).
__device__ __forceinline__ int wrow(int o) { return 4 * (o & 3) + ((o >> 2) & 3) + (o & ~15); }

// Weight unit u of a stage: mode m, input channel i, outputs 4 c .. 4 c + 3
// (c: two bits from u, one from bit 6), so that four lanes read 64 bytes of
// one (mode, i) row and 32 lanes store 8 channels of 4 output groups.
__device__ __forceinline__ void wunit(int u, int &m, int &i, int &c) {
  c = (u & 3) + 4 * ((u >> 6) & 1);
  i = (u >> 2) & (kIC - 1);
  m = u >> 7;
}

// WT: weight unit u of a stage: mode m, output row n, contracted channels
// 4 q .. 4 q + 3 of the stage. Four lanes read 64 bytes of one W row; the
// 8 lanes of one 16-byte store pass cover rows n and n + 8 (wrow 2 apart:
// 48 words, 16 banks mod 32), so their stores hit 32 distinct banks.
__device__ __forceinline__ void wunit_t(int u, int &m, int &n, int &q) {
  const int x = (u >> 2) & 31;
  q = u & 3;
  n = 8 * (x & 1) + ((x >> 1) & 7) + 16 * (x >> 4);
  m = u >> 7;
}

// one spectra unit in flight: two modes of one (b, i) row; complex fp32
// (re, im, re, im) bits, or (HX) two fp16 pairs and the row's exponent
template <bool HX>
struct XReg {
  u32x4 v;
};
template <>
struct XReg<true> {
  uint2 v;
  int e;
};

template <int DT, int MT, int MB, bool HX, bool WT>
__device__ __forceinline__ void cmx_fetch(const ContractArgs &a, int st, int k0, int b0, int o0, int tid,
                                          XReg<HX> (&px)[CmxShape<DT, MT, MB, HX>::XU],
                                          u32x4 (&pw)[CmxShape<DT, MT, MB, HX>::WU]) {
  using S = CmxShape<DT, MT, MB, HX>;
  const int K = a.K, Ci = a.Ci, Co = a.Co, B = a.B;
#pragma unroll
  for (int v = 0; v < S::XU; ++v) {
    const int u = v * S::NT + tid;
    const int row = u / S::UX, c = u % S::UX;  // row = (b, i), i fastest; c: modes 2c, 2c + 1
    const int b = b0 + row / kIC, i = st * kIC + row % kIC, mode = k0 + 2 * c;
    const bool ok = b < B && i < Ci && mode < K;
    if constexpr (HX) {
      const size_t r = ok ? (size_t)b * Ci + i : 0;
      const uint2 t = *reinterpret_cast<const uint2 *>(a.xh16 + (ok ? r * K + mode : 0));
      const int e = a.xexp[r];
      px[v].v = ok ? t : make_uint2(0u, 0u);
      px[v].e = e;
    } else {
      const u32x4 t = *reinterpret_cast<const u32x4 *>(a.xh + (ok ? ((size_t)b * Ci + i) * K + mode : 0));
      px[v].v = ok ? t : u32x4{0u, 0u, 0u, 0u};
    }
  }
#pragma unroll
  for (int v = 0; v < S::WU; ++v) {
    if constexpr (WT) {
      // w[mode][n][c] (Ci % 4 == 0: a 16-byte group is whole or absent)
      int m, nl, q;
      wunit_t(v * S::NT + tid, m, nl, q);
      const int mode = k0 + m, n = o0 + nl, c = st * kIC + 4 * q;
      const bool ok = mode < K && n < Co && c < Ci;
      const u32x4 t = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(a.w) +
                                                       (ok ? (((size_t)mode * Co + n) * Ci + c) * 2 : 0));
      pw[v] = ok ? t : u32x4{0u, 0u, 0u, 0u};
    } else {
      int m, il, c;
      wunit(v * S::NT + tid, m, il, c);
      const int mode = k0 + m, i = st * kIC + il, o = o0 + 4 * c;
      const bool ok = mode < K && i < Ci && o < Co;
      const u32x4 t = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(a.w) +
                                                       (ok ? (((size_t)mode * Ci + i) * Co + o) * 2 : 0));
      pw[v] = ok ? t : u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// split and transpose one stage into fragment rows:
//   xs[mode][part][b][2 i + re/im], ws[mode][part][o][2 i + re/im]
// sb: the batch rows' common exponents (DIRECT)
template <int DT, int MT, int MB, bool HX, bool WT>
__device__ __forceinline__ void cmx_put(uint16_t *xs, uint16_t *ws, int tid,
                                        const XReg<HX> (&px)[CmxShape<DT, MT, MB, HX>::XU],
                                        const u32x4 (&pw)[CmxShape<DT, MT, MB, HX>::WU], const int *sb) {
  using S = CmxShape<DT, MT, MB, HX>;
#pragma unroll
  for (int v = 0; v < S::XU; ++v) {
    const int u = v * S::NT + tid;
    const int row = u / S::UX, c = u % S::UX;
    const int b = row / kIC, i = row % kIC;
    if constexpr (S::DIRECT) {
      // to the row's common scale: times 2^(sb - e) <= 1, exact while the
      // result stays a normal fp16
      const float sc = pow2f(sb[b] - px[v].e);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint32_t h = t ? px[v].v.y : px[v].v.x;
        const float re = (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xffffu)) * sc;
        const float im = (float)__builtin_bit_cast(_Float16, (uint16_t)(h >> 16)) * sc;
        const int m = 2 * c + t;
        reinterpret_cast<uint32_t *>(xs + m * S::XB + xrow<MT>(m, b) * kSP)[i] = f16x2_rne(re, im);
      }
      continue;
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      uint32_t hi, lo;
      if constexpr (HX) {
        // each half converted on its own (see the weight split below)
        const float sc = pow2f(-px[v].e);
        const uint32_t h = t ? px[v].v.y : px[v].v.x;
        const float re = (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xffffu)) * sc;
        const float im = (float)__builtin_bit_cast(_Float16, (uint16_t)(h >> 16)) * sc;
        split_pair(re, im, hi, lo);
      } else {
        split_pair(__uint_as_float(px[v].v[2 * t]), __uint_as_float(px[v].v[2 * t + 1]), hi, lo);
      }
      const int m = 2 * c + t;
      reinterpret_cast<uint32_t *>(xs + (m * 2 + 0) * S::XB + xrow<MT>(m, b) * kSP)[i] = hi;
      reinterpret_cast<uint32_t *>(xs + (m * 2 + 1) * S::XB + xrow<MT>(m, b) * kSP)[i] = lo;
    }
  }
  if constexpr (WT) {
#pragma unroll
    for (int v = 0; v < S::WU; ++v) {
      int m, nl, q;
      wunit_t(v * S::NT + tid, m, nl, q);
      uint16_t *dst = ws + ((m * S::HL) * kOT + wrow(nl)) * kSP + 8 * q;
      if constexpr (S::HL == 2) {
        // fp16 weights in bf16 hi + lo parts, each half converted on its own
        u32x4 hi, lo;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float re = (float)__builtin_bit_cast(_Float16, (uint16_t)(pw[v][t] & 0xffffu));
          const float im = (float)__builtin_bit_cast(_Float16, (uint16_t)(pw[v][t] >> 16));
          uint32_t h, l;
          split_pair(re, im, h, l);
          hi[t] = h;
          lo[t] = l;
        }
        *reinterpret_cast<u32x4 *>(dst) = hi;
        *reinterpret_cast<u32x4 *>(dst + kOT * kSP) = lo;
      } else {
        *reinterpret_cast<u32x4 *>(dst) = pw[v];
      }
    }
    return;
  }
#pragma unroll
  for (int v = 0; v < S::WU; ++v) {
    int m, i, c;
    wunit(v * S::NT + tid, m, i, c);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int o = wrow(4 * c + t);
      if constexpr (S::DIRECT) {
        reinterpret_cast<uint32_t *>(ws + (m * kOT + o) * kSP)[i] = pw[v][t];
      } else if constexpr (DT == DT_F16) {
        // each half converted on its own: reading both lanes of a bit-cast
        // half2 vector here produced wrong values on gfx950
        const float re = (float)__builtin_bit_cast(_Float16, (uint16_t)(pw[v][t] & 0xffffu));
        const float im = (float)__builtin_bit_cast(_Float16, (uint16_t)(pw[v][t] >> 16));
        uint32_t hi, lo;
        split_pair(re, im, hi, lo);
        reinterpret_cast<uint32_t *>(ws + ((m * 2 + 0) * kOT + o) * kSP)[i] = hi;
        reinterpret_cast<uint32_t *>(ws + ((m * 2 + 1) * kOT + o) * kSP)[i] = lo;
      } else {
        reinterpret_cast<uint32_t *>(ws + (m * kOT + o) * kSP)[i] = pw[v][t];
      }
    }
  }
}

// B fragment of output column n = 16 nt + l % 16 = (o, part) from raw
// (Re W, Im W) pairs of four consecutive input channels: part 0 takes
// (Re, -Im), part 1 takes (Im, Re). WT (the weight is conj(W)): part 0 takes
// (Re, Im) as it is, part 1 (-Im, Re).
template <bool WT>
__device__ __forceinline__ u32x4 w_form(u32x4 raw, bool part1) {
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (WT)
      o[j] = part1 ? __builtin_amdgcn_alignbit(raw[j], raw[j], 16) ^ 0x00008000u : raw[j];
    else
      o[j] = part1 ? __builtin_amdgcn_alignbit(raw[j], raw[j], 16) : raw[j] ^ 0x80000000u;
  }
  return o;
}

// Waves per SIMD the register allocation targets: four for eight- and
// sixteen-mode workgroups (16 waves per CU; the fp16-weight split form then
// spills 15 registers and still runs faster than with 4-wave workgroups),
// three (fp16 weights, split in two parts) or four for four-mode ones.
template <int DT, int MB, bool HX>
constexpr int cmx_waves() { return MB >= 8 ? 4 : DT == DT_F16 && !HX ? 3 : 4; }

template <int DT, int MT, int MB, bool HX, bool WT>
__global__ __launch_bounds__(cmx_threads<MB>()) __attribute__((amdgpu_waves_per_eu(cmx_waves<DT, MB, HX>()))) void fno_contract_mx(
    ContractArgs a) {
  using S = CmxShape<DT, MT, MB, HX>;
  extern __shared__ uint16_t sm[];
  uint16_t *xs = sm;
  uint16_t *ws = xs + S::XS;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int K = a.K, Co = a.Co, B = a.B;
  // Workgroup id -> (mode block, batch block, output tile). Consecutive ids
  // go to different XCDs (ids equal mod 8 share one XCD and its L2). Each
  // XCD takes one contiguous range of (mode, batch) blocks, output tiles
  // fastest: the tiles of a block, and neighbouring mode blocks (the two
  // halves of each 128-byte line of spectra), run on one XCD at about the
  // same time, so repeated reads hit its L2.
  const int NO = (Co + kOT - 1) / kOT, NKB = ((K + MB - 1) / MB) * ((B + S::BT - 1) / S::BT);
  const int per = (NKB + 7) / 8;  // blocks per XCD
  const int rest = (int)blockIdx.x >> 3;
  const int tkb = ((int)blockIdx.x & 7) * per + rest / NO;
  if (rest / NO >= per || tkb >= NKB) return;  // padding of the last XCD's range
  const int NK = (K + MB - 1) / MB;
  const int k0 = (tkb % NK) * MB, b0 = (tkb / NK) * S::BT, o0 = (rest % NO) * kOT;
  const int nst = (a.Ci + kIC - 1) / kIC;
  const bool part1 = lane & 1;

  // Stage 0 is requested first, so that its latency overlaps the exponent
  // minimum below.
  XReg<HX> px[S::XU];
  u32x4 pw[S::WU];
  cmx_fetch<DT, MT, MB, HX, WT>(a, 0, k0, b0, o0, tid, px, pw);

  // DIRECT: each batch row's common exponent, the smallest over its planes
  // (the largest plane then fits fp16 and every other is scaled down); the
  // exponents are read eight at a time, clamped in range, so that their loads
  // are in flight together
  int *sbl = reinterpret_cast<int *>(sm + S::LH);
  if constexpr (S::DIRECT) {
    int *part = reinterpret_cast<int *>(sm);  // [NT / BT][BT] partial minima
    constexpr int G = S::NT / S::BT;
    const int bl = tid % S::BT, grp = tid / S::BT, b = b0 + bl;
    const int *xe = a.xexp + (size_t)min(b, B - 1) * a.Ci;
    int e = 1 << 20;
    for (int i0 = grp; i0 < a.Ci; i0 += 8 * G) {
      int t[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) t[j] = xe[min(i0 + j * G, a.Ci - 1)];
#pragma unroll
      for (int j = 0; j < 8; ++j) e = i0 + j * G < a.Ci ? min(e, t[j]) : e;
    }
    part[grp * S::BT + bl] = b < B ? e : (1 << 20);
    __syncthreads();
    if (tid < S::BT) {
      int m = part[tid];
#pragma unroll
      for (int g = 1; g < G; ++g) m = min(m, part[g * S::BT + tid]);
      sbl[tid] = m < (1 << 20) ? m : 0;
    }
    __syncthreads();
  }

  v4f acc[S::MW][MT][4];
#pragma unroll
  for (int mm = 0; mm < S::MW; ++mm)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mm][mt][nt] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int st = 0; st < nst; ++st) {
    cmx_put<DT, MT, MB, HX, WT>(xs, ws, tid, px, pw, sbl);
    if (st + 1 < nst) cmx_fetch<DT, MT, MB, HX, WT>(a, st + 1, k0, b0, o0, tid, px, pw);
    __syncthreads();
#pragma unroll
    for (int mm = 0; mm < S::MW; ++mm) {
      const int m = S::MW * wv + mm;
      u32x4 af[MT][S::XP];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int p = 0; p < S::XP; ++p)
          af[mt][p] = *reinterpret_cast<const u32x4 *>(xs + (m * S::XP + p) * S::XB +
                                                       xrow<MT>(m, mt * 16 + (lane & 15)) * kSP + 8 * (lane >> 4));
#pragma unroll
      for (int nh = 0; nh < 2; ++nh) {  // two halves of the output tiles
        u32x4 bf[2][S::HL];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int p = 0; p < S::HL; ++p)
            bf[t][p] = *reinterpret_cast<const u32x4 *>(
                ws + ((m * S::HL + p) * kOT + wrow((2 * nh + t) * 8 + ((lane & 15) >> 1))) * kSP + 8 * (lane >> 4));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int p = 0; p < S::HL; ++p) bf[t][p] = w_form<WT>(bf[t][p], part1);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            v4f &c = acc[mm][mt][2 * nh + t];
            if constexpr (S::DIRECT) {
              c = mma_f16(af[mt][0], bf[t][0], c);
            } else {
              c = mma_bf(af[mt][0], bf[t][0], c);
              c = mma_bf(af[mt][S::XP - 1], bf[t][0], c);
              if constexpr (S::HL == 2) c = mma_bf(af[mt][0], bf[t][1], c);
            }
          }
      }
    }
    __syncthreads();
  }

  // results -> LDS ys[b][o][8 modes] (re, im) -> rows of 8 modes of Yh, 16
  // batch rows at a time; row pitches of YO and YB floats keep the
  // stores to at most two lanes per bank
  float *ys = reinterpret_cast<float *>(sm);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt > 0) __syncthreads();
#pragma unroll
    for (int mm = 0; mm < S::MW; ++mm)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int n = nt * 16 + (lane & 15), o = n >> 1, part = n & 1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int b = 4 * (lane >> 4) + j;
          ys[b * S::YB + o * S::YO + (S::MW * wv + mm) * 2 + part] = acc[mm][mt][nt][j];
        }
      }
    __syncthreads();
    if constexpr (HX) {
      // groups of four modes of one (b, o) row: largest magnitude ->
      // exponent, fp16 pairs scaled by it (a group cut by K keeps two modes)
      constexpr int GR = MB / 4;                    // groups per row
      constexpr int YG = 16 * kOT * GR / S::NT;     // groups per thread
      const int KQ = (K + 3) >> 2;
#pragma unroll
      for (int v = 0; v < YG; ++v) {
        const int u = v * S::NT + tid;
        const int row = u / GR, c = u % GR;
        const int bl = row / kOT, ol = row % kOT;
        const int b = b0 + mt * 16 + bl, o = o0 + ol, mode = k0 + 4 * c;
        if (b < B && o < Co && mode < K) {
          const float *src = ys + bl * S::YB + ol * S::YO + 8 * c;
          const float4 p0 = *reinterpret_cast<const float4 *>(src), p1 = *reinterpret_cast<const float4 *>(src + 4);
          const float m = fmaxf(fmaxf(fmaxf(fabsf(p0.x), fabsf(p0.y)), fmaxf(fabsf(p0.z), fabsf(p0.w))),
                                fmaxf(fmaxf(fabsf(p1.x), fabsf(p1.y)), fmaxf(fabsf(p1.z), fabsf(p1.w))));
          int e = 0;
          if (m > 0.f) (void)frexpf(m, &e);  // m < 2^e
          // DIRECT: the accumulators hold the true values times 2^sb of the
          // batch row; the stored pairs are the true values times 2^sx
          const int rs = S::DIRECT ? sbl[mt * 16 + bl] : 0;
          const int sx = m > 0.f ? max(-120, min(120, 14 - e + rs)) : 0;
          const float f = pow2f(sx) * pow2f(-rs);
          uint32_t *dst = a.yh16 + ((size_t)b * Co + o) * K + mode;
          const uint2 h0 = make_uint2(f16x2_rne(p0.x * f, p0.y * f), f16x2_rne(p0.z * f, p0.w * f));
          const uint2 h1 = make_uint2(f16x2_rne(p1.x * f, p1.y * f), f16x2_rne(p1.z * f, p1.w * f));
          if ((K & 3) == 0) {
            // whole groups, 16-byte aligned (mode and every row start are
            // multiples of 4): one store
            *reinterpret_cast<uint4 *>(dst) = make_uint4(h0.x, h0.y, h1.x, h1.y);
          } else {
            *reinterpret_cast<uint2 *>(dst) = h0;
            if (mode + 2 < K) *reinterpret_cast<uint2 *>(dst + 2) = h1;
          }
          a.yexp[((size_t)b * Co + o) * KQ + (mode >> 2)] = (signed char)sx;
        }
      }
    } else {
      constexpr int YU = 16 * kOT * MB * 8 / 16 / S::NT;  // 16-byte result units per thread
#pragma unroll
      for (int v = 0; v < YU; ++v) {
        const int u = v * S::NT + tid;
        const int row = u / S::UX, c = u % S::UX;  // row = (b, o); c: modes 2c, 2c + 1
        const int bl = row / kOT, ol = row % kOT;
        const int b = b0 + mt * 16 + bl, o = o0 + ol, mode = k0 + 2 * c;
        if (b < B && o < Co && mode < K)
          *reinterpret_cast<u32x4 *>(a.yh + ((size_t)b * Co + o) * K + mode) =
              *reinterpret_cast<const u32x4 *>(ys + bl * S::YB + ol * S::YO + 4 * c);
      }
    }
  }
}

// -------------------------------------------------------------- launchers

bool contract_mx_supported(int dtype, int Co, int K) {
  return (dtype == DT_F16 || dtype == DT_BF16) && (Co & 3) == 0 && (K & 1) == 0;
}

// Eight-mode workgroups (the tiling the plan's choice of this kernel is
// measured on)
long contract_mx_workgroups(int B, int Co, int K) {
  const long BT = B <= 16 ? 16 : 32;
  return (long)((K + 7) / 8) * ((B + BT - 1) / BT) * ((Co + kOT - 1) / kOT);
}

static size_t contract_mx_lds_bytes(int dtype, int B, int mb, bool hx);

constexpr size_t kLdsMax = 160 * 1024;  // LDS of a CU, the most one workgroup may take

// Modes per workgroup. 16 (one 16-wave workgroup per CU) where that still
// gives every CU a workgroup and its LDS fits: at 256^2 (B = 32, 64
// channels, 32 x 32 modes) 25.0 -> 23.9 us fp16 and 22.9 -> 20.0 us bf16 on
// the half exchange against 8 modes; not for the fp16 adjoint, which
// measured 22.4 -> 22.9 us. Else 8 unless that leaves resident slots empty
// (two eight-mode workgroups fit on each CU); then 4, which doubles the
// workgroups. Measured: the FNO2d layer (B = 20, 64 -> 64 channels, modes
// 24 x 24: 288 eight-mode workgroups) runs faster with 4 (16.1 against 17.4
// us with 8), the 256^2 layer with 8 faster than with 4 (25.0 against 31.1).
static int cmx_modes(int dtype, int B, int Co, int K, bool hx, bool wt) {
  const long BT = B <= 16 ? 16 : 32;
  const long wg16 = (long)((K + 15) / 16) * ((B + BT - 1) / BT) * ((Co + kOT - 1) / kOT);
  if (!(wt && dtype == DT_F16) && wg16 >= 256 && contract_mx_lds_bytes(dtype, B, 16, hx) <= kLdsMax) return 16;
  return contract_mx_workgroups(B, Co, K) < 512 ? 4 : 8;
}

template <int DT, bool HX, bool WT>
static const void *contract_mx_kernel_dt(int B, int mb) {
  const bool one = B <= 16;
  if (mb == 4)
    return one ? (const void *)fno_contract_mx<DT, 1, 4, HX, WT> : (const void *)fno_contract_mx<DT, 2, 4, HX, WT>;
  if (mb == 16)
    return one ? (const void *)fno_contract_mx<DT, 1, 16, HX, WT> : (const void *)fno_contract_mx<DT, 2, 16, HX, WT>;
  return one ? (const void *)fno_contract_mx<DT, 1, 8, HX, WT> : (const void *)fno_contract_mx<DT, 2, 8, HX, WT>;
}

template <int DT>
static const void *contract_mx_kernel_d(int B, int mb, bool hx, bool wt) {
  if (hx) return wt ? contract_mx_kernel_dt<DT, true, true>(B, mb) : contract_mx_kernel_dt<DT, true, false>(B, mb);
  return wt ? contract_mx_kernel_dt<DT, false, true>(B, mb) : contract_mx_kernel_dt<DT, false, false>(B, mb);
}

static const void *contract_mx_kernel(int dtype, int B, int mb, bool hx, bool wt) {
  if (dtype == DT_F16) return contract_mx_kernel_d<DT_F16>(B, mb, hx, wt);
  if (dtype == DT_BF16) return contract_mx_kernel_d<DT_BF16>(B, mb, hx, wt);
  return nullptr;
}

static size_t contract_mx_lds_bytes(int dtype, int B, int mb, bool hx) {
  const bool direct = hx && dtype == DT_F16;
  const int BT = B <= 16 ? 16 : 32, XP = direct ? 1 : 2, HL = dtype == DT_F16 && !direct ? 2 : 1;
  const size_t stage = ((size_t)mb * XP * BT * kSP + (size_t)mb * HL * kOT * kSP) * 2;
  const size_t out = (size_t)16 * (kOT * (2 * mb + 4) + 4) * 4;
  return std::max(std::max(stage, out), (size_t)mb * 64 * 4) + (direct ? BT * 4 : 0);
}

size_t contract_mx_lds_bytes(int dtype, int B) {
  size_t m = 0;
  for (int mb : {4, 8, 16})
    for (bool hx : {false, true}) {
      const size_t l = contract_mx_lds_bytes(dtype, B, mb, hx);
      if (l <= kLdsMax) m = std::max(m, l);
    }
  return m;
}

hipError_t contract_mx_prepare(int dtype, int B) {
  for (int mb : {4, 8, 16})
    for (bool hx : {false, true})
      for (bool wt : {false, true}) {
        const size_t lds = contract_mx_lds_bytes(dtype, B, mb, hx);
        if (mb == 16 && lds > kLdsMax) continue;  // never chosen
        const void *k = contract_mx_kernel(dtype, B, mb, hx, wt);
        if (!k) return hipErrorInvalidValue;
        const hipError_t e = raise_lds_cap(k, lds);
        if (e != hipSuccess) return e;
      }
  return hipSuccess;
}

bool contract_mx_wt_supported(int Ci) { return (Ci & 3) == 0; }

hipError_t launch_contract_mx(const ContractArgs &a, int dtype, hipStream_t s, bool wt) {
  FNO_BOUNDS(check_contract(a, dtype, true);)
  const int mb = cmx_modes(dtype, a.B, a.Co, a.K, a.xh16 != nullptr, wt);
  const void *k = contract_mx_kernel(dtype, a.B, mb, a.xh16 != nullptr, wt);
  if (!k || (wt && !contract_mx_wt_supported(a.Ci))) return hipErrorInvalidValue;
  const int BT = a.B <= 16 ? 16 : 32;
  const long nkb = (long)((a.K + mb - 1) / mb) * ((a.B + BT - 1) / BT), no = (a.Co + kOT - 1) / kOT;
  const long n = (nkb + 7) / 8 * 8 * no;
  if (n > 0x7fffffffL) return hipErrorInvalidValue;
  dim3 grid((unsigned)n);
  void *args[] = {(void *)&a};
  return hipLaunchKernel(k, grid, dim3(mb * 64), args, contract_mx_lds_bytes(dtype, a.B, mb, a.xh16 != nullptr), s);
}

}  // namespace fno
