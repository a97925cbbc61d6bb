// plane_mfma.hip - plane transforms of fp16 / bf16 planes as two streamed
// matrix-core contractions each way.
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
// All four run on v_mfma_f32_16x16x32_{f16,bf16} with fp32 accumulation.
//
// Rows are streamed in rounds of 64. The column product of one round uses
// the same 64-row twiddle block for every round: the round offset h0 only
// multiplies mode q by e^{-+2 pi i kx(q) h0 / H}, which is applied to the
// per-round partial sums (forward) or to the spectra (inverse) on the VALU.
// So a workgroup holds one 64-row stage of x or y, one round of R or Z, and
// its twiddle fragments in registers: about 45-55 KB of LDS, two workgroups
// of 8 waves per CU.
//
// Precision. x (fp16) is exact as an MFMA operand; bf16 x is multiplied by a
// two-term bf16 split of T. R, Z and the spectra are rounded to fp16 after a
// power-of-two scale derived from a bound (the round's max |x| times W, or
// the plane's max |Y| times 4 m1), which keeps every fp16 operand below 2^15
// and far above the subnormal range for data of any sensible magnitude; the
// scale is undone in fp32. Twiddles are rounded to fp16.
//
// One fragment of v_mfma_f32_16x16x32 (A: 16 x 32, B: 32 x 16): lane l holds
// row / column l % 16 and the eight consecutive k = 8 (l / 16) .. +7;
// accumulator register j of lane l holds row 4 (l / 16) + j, column l % 16.

#include "common.hpp"

namespace fno {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));

constexpr int kGT = 512;   // threads per workgroup (8 waves)
constexpr int kRows = 64;  // rows per round
constexpr int kRBP = 136;  // halves per row of a B-operand round buffer (128 + pad)
constexpr int kZBP = 72;   // halves per row of the inverse Z buffer (64 + pad)

__device__ __forceinline__ v4f mma(u32x4 a, u32x4 b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c, 0, 0, 0);
}

__device__ __forceinline__ v4f mma_bf(u32x4 a, u32x4 b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, a), __builtin_bit_cast(b8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint16_t h16(float v) { return __builtin_bit_cast(uint16_t, (_Float16)v); }

__device__ __forceinline__ uint32_t h16x2(float lo, float hi) {
  return (uint32_t)h16(lo) | ((uint32_t)h16(hi) << 16);
}

// largest magnitude field of eight packed 16-bit floats (sign cleared); for
// finite fp16 and bf16 values the unsigned order of these bits is the order
// of the magnitudes
__device__ __forceinline__ uint32_t absmax_bits(u32x4 v) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m = max(m, v[i] & 0x7fffu);
    m = max(m, (v[i] >> 16) & 0x7fffu);
  }
  return m;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// 2^e as an fp32 with e clamped to a range where it and 2^-e are normal
__device__ __forceinline__ float pow2f(int e) {
  e = max(-120, min(120, e));
  return __uint_as_float((uint32_t)(e + 127) << 23);
}

// ------------------------------------------------------------------ forward

template <int KB>
__device__ __forceinline__ void fwd_fetch(const u32x4 *xp, int r, int tid, u32x4 (&p)[KB / 2]) {
  constexpr int WU = 4 * KB;  // 16-byte units per row
  const u32x4 *src = xp + (size_t)r * kRows * WU + tid;
#pragma unroll
  for (int v = 0; v < KB / 2; ++v) p[v] = src[v * kGT];
}

struct FwdShape {
  int H, m1, m2, NT, MT, NN, lgW;
};

// One round of 64 rows: stage them, row product into R (fp16, scaled), then
// the column product of R against the 64-row twiddle block, phase-shifted
// and accumulated into X.
template <int DT, int KB>
__device__ __forceinline__ void fwd_round(int r, int rounds, const FwdShape &s, u32x4 (&p)[KB / 2],
                                          const u32x4 *xp, u32x4 *stage, uint16_t *rb, const float2 *twh,
                                          uint32_t *mxs, const u32x4 (&th)[KB],
                                          const u32x4 (&tl)[DT == DT_BF16 ? KB : 1], const u32x4 (&ef)[4],
                                          float2 (&X)[2][2]) {
  constexpr bool BF = DT == DT_BF16;
  constexpr int WU = 4 * KB, PITCH = WU + 1;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

  uint32_t mb = 0;
#pragma unroll
  for (int v = 0; v < KB / 2; ++v) {
    const int e = v * kGT + tid;
    const int row = e / WU, cu = e - row * WU;
    stage[row * PITCH + cu] = p[v];
    mb = max(mb, absmax_bits(p[v]));
  }
  mb = wave_max_u32(mb);
  if (lane == 0) mxs[(r & 1) * 8 + wv] = mb;
  if (r + 2 < rounds) fwd_fetch<KB>(xp, r + 2, tid, p);
  __syncthreads();

  // scale: |R| <= W max|x| < 2^(e + lgW); R * 2^(15 - e - lgW) < 2^15
  uint32_t mall = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) mall = max(mall, mxs[(r & 1) * 8 + i]);
  int e;
  if constexpr (BF) e = (int)max(mall >> 7, 1u) - 126;
  else e = (int)max(mall >> 10, 1u) - 14;
  const int se = mall ? 15 - e - s.lgW : 0;
  const float sc = pow2f(se), isc = pow2f(-se);

  // row product: column tile nt of R for the stripes of this wave
  const int nt = wv % s.NT;
  for (int st = wv / s.NT; st < 4; st += 8 / s.NT) {
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    const u32x4 *ar = stage + (st * 16 + (lane & 15)) * PITCH + (lane >> 4);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const u32x4 av = ar[kb * 4];
      if constexpr (BF) {
        acc = mma_bf(av, th[kb], acc);
        acc = mma_bf(av, tl[kb], acc);
      } else {
        acc = mma(av, th[kb], acc);
      }
    }
    const int c = nt * 16 + (lane & 15);
    if (c < 2 * s.m2) {
      uint16_t *dst = rb + (c >> 1) * kRBP + 2 * (st * 16 + 4 * (lane >> 4)) + (c & 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[2 * j] = h16(acc[j] * sc);
    }
  }
  __syncthreads();

  // column product: m-tile wv (modes q0, q0 + 1 per lane), all ky tiles
  if (wv < s.MT) {
    const int q0 = 8 * wv + 2 * (lane >> 4);
    float2 ph[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int q = q0 + t;
      const int kx = q < s.m1 ? q : s.H - 2 * s.m1 + q;
      ph[t] = twh[(kx * kRows * r) & (s.H - 1)];
    }
#pragma unroll
    for (int nn = 0; nn < 2; ++nn) {
      if (nn < s.NN) {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
        const u32x4 *br = reinterpret_cast<const u32x4 *>(rb + (nn * 16 + (lane & 15)) * kRBP) + (lane >> 4);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) acc = mma(ef[kb], br[kb * 4], acc);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const float yr = acc[2 * t] * isc, yi = acc[2 * t + 1] * isc;
          X[nn][t].x += yr * ph[t].x - yi * ph[t].y;
          X[nn][t].y += yr * ph[t].y + yi * ph[t].x;
        }
      }
    }
  }
}

template <int DT, int KB>
__global__ __launch_bounds__(kGT) void fno_fwd_plane_mx(PlaneMxFwdArgs a) {
  constexpr bool BF = DT == DT_BF16;
  constexpr int W = 32 * KB, WU = 4 * KB, PITCH = WU + 1;
  extern __shared__ u32x4 lds[];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const FwdShape s{a.H, a.m1, a.m2, a.nt, a.mt, a.nn, a.lgW};
  u32x4 *stage = lds;                                                    // [64][PITCH]
  uint16_t *rb = reinterpret_cast<uint16_t *>(stage + kRows * PITCH);    // [32][kRBP]
  float2 *twh = reinterpret_cast<float2 *>(rb + 32 * kRBP);              // [H]
  uint32_t *mxs = reinterpret_cast<uint32_t *>(twh + s.H);               // [2][8]
  for (int v = tid; v < s.H; v += kGT) twh[v] = a.tw_h[v];

  const int plane = blockIdx.x;
  const u32x4 *xp = reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(a.x) + (size_t)plane * s.H * W);

  // row twiddles of this wave's column tile; column twiddles of its m-tile
  const int nt = wv % s.NT;
  u32x4 th[KB], tl[BF ? KB : 1];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    th[kb] = reinterpret_cast<const u32x4 *>(a.tf)[((size_t)nt * KB + kb) * 64 + lane];
    if constexpr (BF) tl[kb] = reinterpret_cast<const u32x4 *>(a.tf_lo)[((size_t)nt * KB + kb) * 64 + lane];
  }
  const int mt = wv < s.MT ? wv : 0;
  u32x4 ef[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) ef[kb] = reinterpret_cast<const u32x4 *>(a.ef)[((size_t)mt * 4 + kb) * 64 + lane];

  float2 X[2][2];
#pragma unroll
  for (int nn = 0; nn < 2; ++nn)
#pragma unroll
    for (int t = 0; t < 2; ++t) X[nn][t] = make_float2(0.f, 0.f);

  const int rounds = s.H / kRows;
  u32x4 pa[KB / 2], pb[KB / 2];
  fwd_fetch<KB>(xp, 0, tid, pa);
  if (rounds > 1) fwd_fetch<KB>(xp, 1, tid, pb);
  __syncthreads();
  for (int r = 0; r < rounds; r += 2) {
    fwd_round<DT, KB>(r, rounds, s, pa, xp, stage, rb, twh, mxs, th, tl, ef, X);
    if (r + 1 < rounds) fwd_round<DT, KB>(r + 1, rounds, s, pb, xp, stage, rb, twh, mxs, th, tl, ef, X);
  }

  if (wv < s.MT) {
    const int K = 2 * s.m1 * s.m2;
    float2 *op = a.out + (size_t)plane * K;
#pragma unroll
    for (int nn = 0; nn < 2; ++nn) {
      const int ky = nn * 16 + (lane & 15);
      if (nn < s.NN && ky < s.m2) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int q = 8 * wv + 2 * (lane >> 4) + t;
          if (q < 2 * s.m1) op[q * s.m2 + ky] = make_float2(X[nn][t].x * a.scale, X[nn][t].y * a.scale);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ inverse

template <int DT, int KB>
__global__ __launch_bounds__(kGT) void fno_inv_plane_mx(PlaneMxInvArgs a) {
  constexpr int W = 32 * KB, WU = 4 * KB, PITCH = WU + 1;
  constexpr int NTW = W / 16;                  // output column tiles
  constexpr int NBW = NTW >= 8 ? NTW / 8 : 1;  // column tiles per wave
  constexpr int NY = 4;                        // spectra values per thread (K <= 2048)
  extern __shared__ u32x4 lds[];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int H = a.H, m1 = a.m1, m2 = a.m2, NN = a.nn, KB1 = a.kb1;
  const int K = 2 * m1 * m2;
  u32x4 *ostage = lds;                                                      // [64][PITCH]
  uint16_t *yb = reinterpret_cast<uint16_t *>(ostage + kRows * PITCH);      // [32][kRBP]
  uint16_t *zb = yb + 32 * kRBP;                                            // [64][kZBP]
  float2 *twh = reinterpret_cast<float2 *>(zb + kRows * kZBP);              // [H]
  float *ymx = reinterpret_cast<float *>(twh + H);                          // [8]

  for (int v = tid; v < 32 * kRBP / 2; v += kGT) reinterpret_cast<uint32_t *>(yb)[v] = 0u;
  for (int v = tid; v < H; v += kGT) twh[v] = a.tw_h[v];

  const int plane = blockIdx.x;
  const float2 *ip = a.in + (size_t)plane * K;
  float2 yv[NY];
  float mloc = 0.f;
#pragma unroll
  for (int i = 0; i < NY; ++i) {
    const int v = tid + i * kGT;
    const bool ok = v < K;
    const float2 t = ip[ok ? v : 0];
    yv[i] = ok ? t : make_float2(0.f, 0.f);
    mloc = fmaxf(mloc, fmaxf(fabsf(yv[i].x), fabsf(yv[i].y)));
  }
  mloc = wave_max_f32(mloc);
  if (lane == 0) ymx[wv] = mloc;

  // E' fragments of m-tile wv (rows j = 8 wv .. 8 wv + 7, both parts)
  u32x4 ef[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const u32x4 t = reinterpret_cast<const u32x4 *>(a.ef)[((size_t)wv * KB1 + (kb < KB1 ? kb : 0)) * 64 + lane];
    ef[kb] = kb < KB1 ? t : u32x4{0u, 0u, 0u, 0u};
  }
  // T' fragments of this wave's output column tiles
  u32x4 tb[NBW][2];
#pragma unroll
  for (int b = 0; b < NBW; ++b) {
    const int ntl = NTW >= 8 ? wv + 8 * b : wv % NTW;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const u32x4 t = reinterpret_cast<const u32x4 *>(a.tb)[((size_t)ntl * NN + (kb < NN ? kb : 0)) * 64 + lane];
      tb[b][kb] = kb < NN ? t : u32x4{0u, 0u, 0u, 0u};
    }
  }
  __syncthreads();

  // |Z| <= sum_q (|Re Y| + |Im Y|) <= 4 m1 max|Y| < 2^(e + lg4m1)
  float ym = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ym = fmaxf(ym, ymx[i]);
  int e = 0;
  if (ym > 0.f) (void)frexpf(ym, &e);
  const int se = ym > 0.f ? 15 - e - a.lg4m1 : 0;
  const float sc = pow2f(se), isc = pow2f(-se);

  uint4 *yp = reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(a.y) + (size_t)plane * H * W);
  const int rounds = H / kRows;
  for (int r = 0; r < rounds; ++r) {
    // spectra of the round: Y[q][ky] e^{+2 pi i kx(q) h0 / H}, scaled, fp16
#pragma unroll
    for (int i = 0; i < NY; ++i) {
      const int v = tid + i * kGT;
      if (v < K) {
        const int q = v / m2, ky = v - q * m2;
        const int kx = q < m1 ? q : H - 2 * m1 + q;
        const float2 w = twh[(kx * kRows * r) & (H - 1)];  // e^{-i theta}
        const float zr = (yv[i].x * w.x + yv[i].y * w.y) * sc;
        const float zi = (yv[i].y * w.x - yv[i].x * w.y) * sc;
        reinterpret_cast<uint32_t *>(yb + ky * kRBP)[q] = h16x2(zr, zi);
      }
    }
    __syncthreads();

    // Z = E' Y for rows j = 8 wv .. +7 (m-tile wv), all ky tiles; fp16 into zb
#pragma unroll
    for (int nn = 0; nn < 2; ++nn) {
      if (nn < NN) {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
        const u32x4 *br = reinterpret_cast<const u32x4 *>(yb + (nn * 16 + (lane & 15)) * kRBP) + (lane >> 4);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          if (kb < KB1) acc = mma(ef[kb], br[kb * 4], acc);
        const int j0 = 8 * wv + 2 * (lane >> 4), ky = nn * 16 + (lane & 15);
        reinterpret_cast<uint32_t *>(zb + j0 * kZBP)[ky] = h16x2(acc[0], acc[1]);
        reinterpret_cast<uint32_t *>(zb + (j0 + 1) * kZBP)[ky] = h16x2(acc[2], acc[3]);
      }
    }
    __syncthreads();

    // y = Z T' for this wave's tiles, unscaled and rounded into the out stage
    uint16_t *os = reinterpret_cast<uint16_t *>(ostage);
#pragma unroll
    for (int b = 0; b < NBW; ++b) {
      const int ntl = NTW >= 8 ? wv + 8 * b : wv % NTW;
      const int mstep = NTW >= 8 ? 1 : 8 / NTW;
      for (int mtl = NTW >= 8 ? 0 : wv / NTW; mtl < 4; mtl += mstep) {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
        const u32x4 *ar = reinterpret_cast<const u32x4 *>(zb + (mtl * 16 + (lane & 15)) * kZBP) + (lane >> 4);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          if (kb < NN) acc = mma(ar[kb * 4], tb[b][kb], acc);
        uint16_t *dst = os + (mtl * 16 + 4 * (lane >> 4)) * PITCH * 8 + ntl * 16 + (lane & 15);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float v = acc[j] * isc;
          dst[j * PITCH * 8] = DT == DT_F16 ? h16(v) : (uint16_t)f32_to_bf16(v);
        }
      }
    }
    __syncthreads();

    // 64 rows x W halves: coalesced 16-byte stores
#pragma unroll
    for (int v = 0; v < KB / 2; ++v) {
      const int e2 = v * kGT + tid;
      const int row = e2 / WU, cu = e2 - row * WU;
      yp[(size_t)r * kRows * WU + e2] = reinterpret_cast<const uint4 *>(ostage)[row * PITCH + cu];
    }
  }
}

// --------------------------------------------------------------- launchers

bool mx_supported(int H, int W, int m1, int m2, int dtype) {
  return (dtype == DT_F16 || dtype == DT_BF16) && H >= kRows && H <= 256 && W >= 64 && W <= 256 && m1 <= 32 &&
         m2 <= 32 && 2 * m1 <= H;
}

int mx_ntiles(int m2) { return m2 <= 8 ? 1 : m2 <= 16 ? 2 : 4; }

size_t mx_fwd_lds_bytes(int H, int W) {
  return (size_t)kRows * (W / 8 + 1) * 16 + (size_t)32 * kRBP * 2 + (size_t)H * 8 + 64;
}

size_t mx_inv_lds_bytes(int H, int W) {
  return (size_t)kRows * (W / 8 + 1) * 16 + (size_t)32 * kRBP * 2 + (size_t)kRows * kZBP * 2 + (size_t)H * 8 + 32;
}

template <int DT>
static const void *mx_kernel_dt(bool fwd, int W) {
  switch (W) {
    case 64: return fwd ? (const void *)fno_fwd_plane_mx<DT, 2> : (const void *)fno_inv_plane_mx<DT, 2>;
    case 128: return fwd ? (const void *)fno_fwd_plane_mx<DT, 4> : (const void *)fno_inv_plane_mx<DT, 4>;
    case 256: return fwd ? (const void *)fno_fwd_plane_mx<DT, 8> : (const void *)fno_inv_plane_mx<DT, 8>;
  }
  return nullptr;
}

static const void *mx_kernel(bool fwd, int W, int dtype) {
  if (dtype == DT_F16) return mx_kernel_dt<DT_F16>(fwd, W);
  if (dtype == DT_BF16) return mx_kernel_dt<DT_BF16>(fwd, W);
  return nullptr;
}

hipError_t mx_prepare(bool fwd, int W, int dtype, size_t lds) {
  const void *k = mx_kernel(fwd, W, dtype);
  if (!k) return hipErrorInvalidValue;
  return hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

hipError_t launch_plane_mx_fwd(const PlaneMxFwdArgs &a, int dtype, size_t lds, hipStream_t s) {
  const void *k = mx_kernel(true, a.W, dtype);
  if (!k) return hipErrorInvalidValue;
  void *args[] = {(void *)&a};
  return hipLaunchKernel(k, dim3(a.nplanes), dim3(kGT), args, lds, s);
}

hipError_t launch_plane_mx_inv(const PlaneMxInvArgs &a, int dtype, size_t lds, hipStream_t s) {
  const void *k = mx_kernel(false, a.W, dtype);
  if (!k) return hipErrorInvalidValue;
  void *args[] = {(void *)&a};
  return hipLaunchKernel(k, dim3(a.nplanes), dim3(kGT), args, lds, s);
}

}  // namespace fno
