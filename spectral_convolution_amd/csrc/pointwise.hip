// pointwise.hip - per-pixel channel mixing for the full FNO2d network.
//
// The network around the spectral layer (TurboFNO write-up, sections 1 and
// 4.3: the fused layer replaces the spectral convolution inside an FNO
// model): a lifting Linear, per block a 1x1 convolution added to the
// spectral branch followed by GELU, and a two-Linear projection with GELU
// between them.
//
// Both kernels are per-pixel GEMMs on v_mfma_f32_16x16x4f32 in the natural
// [B][C][pixels] layout: the B operand of the MFMA holds one channel x 16
// pixels per 16-lane group, so every activation load and store is a
// contiguous run of pixels of one channel. A lane owns 4 consecutive pixels
// (one per MFMA "t"), 16 lanes span 64 pixels. Weights are converted to fp32
// once per workgroup into LDS. Accumulation is fp32; outputs are rounded
// (RNE) to the storage dtype.

#include <algorithm>

#include "common.hpp"

namespace fno {

// y[b][o][p] = act(sum_i A[o][i] x[b][i][p] + bias[o] + add[b][o][p])
struct MixArgs {
  const void *x, *A, *bias, *add;
  void *y;
  int B, I, O;
  long P;
  int act;  // 0: none, 1: GELU
};

// y[b][c][p] = sum_j Q2[c][j] GELU(sum_i Q1[j][i] x[b][i][p] + q1[j]) + q2[c]
struct ProjArgs {
  const void *x, *Q1, *q1, *Q2, *q2;
  void *y;
  int B, I, J, C;
  long P;
};

template <int DT>
__device__ __forceinline__ float load1(const void *p, size_t i) {
  if constexpr (DT == DT_F32) return reinterpret_cast<const float *>(p)[i];
  else if constexpr (DT == DT_F16) return (float)reinterpret_cast<const _Float16 *>(p)[i];
  else return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(p)[i] << 16);
}

// Four consecutive elements p[base + p0 .. +3] of a row of P elements, zeros
// where ok is false or past the row's end. The loads are unconditional (a
// masked lane reads element 0 of the buffer and discards it) so that the
// compiler can keep several of them in flight. AL: P is a multiple of 4, so a
// run is either whole or entirely past the end and one vector load serves it.
template <int DT, bool AL>
__device__ __forceinline__ void load4(const void *p, size_t base, long p0, long P, bool ok, float (&v)[4]) {
  if constexpr (AL) {
    const bool in = ok && p0 < P;
    const size_t i = in ? base + (size_t)p0 : 0;
    float u[4];
    if constexpr (DT == DT_F32) {
      const float4 q = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(p) + i);
      u[0] = q.x; u[1] = q.y; u[2] = q.z; u[3] = q.w;
    } else {
      const uint2 q = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(p) + i);
      if constexpr (DT == DT_F16) {
        const half2_t h0 = __builtin_bit_cast(half2_t, q.x), h1 = __builtin_bit_cast(half2_t, q.y);
        u[0] = (float)h0.x; u[1] = (float)h0.y; u[2] = (float)h1.x; u[3] = (float)h1.y;
      } else {
        u[0] = __uint_as_float(q.x << 16); u[1] = __uint_as_float(q.x & 0xffff0000u);
        u[2] = __uint_as_float(q.y << 16); u[3] = __uint_as_float(q.y & 0xffff0000u);
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) v[t] = in ? u[t] : 0.f;
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bool in = ok && p0 + t < P;
      const float u = load1<DT>(p, in ? base + (size_t)(p0 + t) : 0);
      v[t] = in ? u : 0.f;
    }
  }
}

template <int DT>
__device__ __forceinline__ void store4(void *p, size_t i, int n, bool al, const float (&v)[4]) {
  if (n >= 4 && al) {
    store_pair<DT>(p, i, v[0], v[1]);
    store_pair<DT>(p, i + 2, v[2], v[3]);
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t < n) {
        if constexpr (DT == DT_F32) reinterpret_cast<float *>(p)[i + t] = v[t];
        else if constexpr (DT == DT_F16) reinterpret_cast<_Float16 *>(p)[i + t] = (_Float16)v[t];
        else reinterpret_cast<uint16_t *>(p)[i + t] = (uint16_t)f32_to_bf16(v[t]);
      }
    }
  }
}

__device__ __forceinline__ float gelu(float v) { return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f)); }

// GELU for the half-precision kernels, whose outputs are rounded to 11 (fp16)
// or 8 (bf16) significant bits: erf from Abramowitz & Stegun, Handbook of
// Mathematical Functions, formula 7.1.28, erf(x) = 1 - (1 + a1 x + ... +
// a6 x^6)^-16 for x >= 0 (absolute error below 3e-7; evaluated in fp32 it
// stays below 2e-6), odd symmetry for x < 0. With r = 1 - erf(|v| / sqrt 2),
// GELU(v) = max(v, 0) - |v| r / 2. One reciprocal on the transcendental
// unit; formula 7.1.26 needs an exponential as well, which made the
// projection (128 hidden GELUs per pixel) 21 us slower at B = 20, 256^2.
__device__ __forceinline__ float gelu_half(float v) {
  const float x = fabsf(v) * 0.70710678118654752f;
  float p = fmaf(0.0000430638f, x, 0.0002765672f);
  p = fmaf(p, x, 0.0001520143f);
  p = fmaf(p, x, 0.0092705272f);
  p = fmaf(p, x, 0.0422820123f);
  p = fmaf(p, x, 0.0705230784f);
  p = fmaf(p, x, 1.0f);
  p = p * p;  // ^16 by four squarings; overflows to inf for large x, so r = 0
  p = p * p;
  p = p * p;
  p = p * p;
  const float r = __builtin_amdgcn_rcpf(p);
  return fmaf(-0.5f * fabsf(v), r, fmaxf(v, 0.0f));
}

static constexpr int kPwThreads = 256;
static constexpr int kMaxI = 128;   // input channels held per workgroup
static constexpr int kOB = 64;      // output channels per workgroup (4 MFMA row tiles)

// Rows of A (o0 .. o0+63) x all I input channels, fp32, padded to a multiple
// of 4 channels with zeros: [kOB][Ipad].
template <int DT>
__device__ void stage_weights(const void *A, int O, int I, int o0, int Ipad, float *w) {
  for (int v = threadIdx.x; v < kOB * Ipad; v += kPwThreads) {
    const int o = v / Ipad, i = v - o * Ipad;
    w[v] = (o0 + o < O && i < I) ? load1<DT>(A, (size_t)(o0 + o) * I + i) : 0.f;
  }
}

template <int DT, bool AL>
__global__ __launch_bounds__(kPwThreads) void fno_channel_mix(MixArgs a) {
  __shared__ float w[kOB * kMaxI];
  __shared__ float bias[kOB];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int o0 = blockIdx.y * kOB, b = blockIdx.z;
  const int I = a.I, O = a.O;
  const long P = a.P;
  const int Ipad = (I + 3) & ~3;
  stage_weights<DT>(a.A, O, I, o0, Ipad, w);
  for (int v = threadIdx.x; v < kOB; v += kPwThreads)
    bias[v] = (a.bias && o0 + v < O) ? load1<DT>(a.bias, o0 + v) : 0.f;
  __syncthreads();

  const int kr = lane >> 4, n = lane & 15;
  const size_t xb = (size_t)b * I * P, yb = (size_t)b * O * P;
  const long ntiles = (P + 63) / 64;
  for (long tile = (long)blockIdx.x * 4 + wv; tile < ntiles; tile += (long)gridDim.x * 4) {
    const long p0 = tile * 64 + 4 * n;
    v4f acc[4][4];
#pragma unroll
    for (int mo = 0; mo < 4; ++mo)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[mo][t] = v4f{0.f, 0.f, 0.f, 0.f};
    // channel k0 + kr, fetched one step ahead of its MFMAs
    float xn[4];
    load4<DT, AL>(a.x, xb + (size_t)(kr < I ? kr : 0) * P, p0, P, kr < I, xn);
    for (int k0 = 0; k0 < Ipad; k0 += 4) {
      const int i = k0 + kr, inext = i + 4;
      float xv[4] = {xn[0], xn[1], xn[2], xn[3]};
      load4<DT, AL>(a.x, xb + (size_t)(inext < I ? inext : 0) * P, p0, P, inext < I, xn);
#pragma unroll
      for (int mo = 0; mo < 4; ++mo) {
        const float av = w[(16 * mo + n) * Ipad + i];
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[mo][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, xv[t], acc[mo][t], 0, 0, 0);
      }
    }
    // accumulator register j of lane l: row 4*(l/16) + j, column l%16
    float ad[4][4][4];
#pragma unroll
    for (int mo = 0; mo < 4; ++mo)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int o = o0 + 16 * mo + 4 * kr + j;
        load4<DT, AL>(a.add ? a.add : a.x, yb + (size_t)(o < O ? o : 0) * P, p0, P, a.add && o < O, ad[mo][j]);
      }
#pragma unroll
    for (int mo = 0; mo < 4; ++mo)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ol = 16 * mo + 4 * kr + j, o = o0 + ol;
        if (o >= O || p0 >= P) continue;
        float v[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          v[t] = acc[mo][t][j] + bias[ol] + ad[mo][j][t];
          if (a.act == 1) v[t] = gelu(v[t]);
        }
        store4<DT>(a.y, yb + (size_t)o * P + p0, (int)min((long)4, P - p0), AL, v);
      }
  }
}

// ------------------------------------------- half-precision channel mix
//
// fp16 / bf16 storage: the products of two storage values are exact in
// fp32, so the per-pixel GEMM runs on v_mfma_f32_16x16x32_{f16,bf16} with
// fp32 accumulation (16x the fp32 matrix rate) at no cost in accuracy. The
// operands need the channels contiguous per lane while the activations are
// pixel-contiguous per channel, so a workgroup stages a tile of Ipad
// channels x 256 pixels in LDS ([i][p], coalesced 16-byte row loads of the
// next tile in flight while the current one is multiplied) and builds the
// A fragments from it. Orientation D[p][o] = x^T W^T: the A operand is 16
// pixels x 32 channels, the B operand 32 channels x 16 outputs (rows of W,
// held in registers for the whole kernel). Wave w owns pixels 64 w ..
// 64 w + 63 of the tile and all 64 output channels of the workgroup. The
// fp32 results (plus bias) go through an LDS stage, 32 output channels at a
// time, so that the add input, the fp32 add and GELU, and the output run
// along whole rows with 16-byte accesses (8 rows x 128 contiguous bytes per
// wave instruction); the add input is requested before the products and the
// next tile's channels while they run. Needs
// P % 8 == 0 and at most 64 input channels (wider inputs would spill
// registers).

typedef unsigned pw_u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 pw_h8 __attribute__((ext_vector_type(8)));
typedef __bf16 pw_b8 __attribute__((ext_vector_type(8)));

constexpr int kMxPx = 256;              // pixels per workgroup tile
constexpr int kMxPitch = kMxPx + 4;     // halves per staged channel row: the four lane groups of a
                                        // fragment read (rows 8 apart) start 64 banks apart

template <int DT>
__device__ __forceinline__ v4f pw_mma(pw_u32x4 a, pw_u32x4 b, v4f c) {
  if constexpr (DT == DT_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(pw_h8, a), __builtin_bit_cast(pw_h8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(pw_b8, a), __builtin_bit_cast(pw_b8, b), c, 0, 0, 0);
}

// one tile of x rows into registers: unit u = (channel u / 32, 8 pixels at
// 8 (u % 32)); channels past I and pixels past P read as zeros
template <int KB>
__device__ __forceinline__ void mixmx_fetch(const uint16_t *xb, int I, long P, long pc, int tid,
                                            pw_u32x4 (&r)[KB * 4]) {
#pragma unroll
  for (int v = 0; v < KB * 4; ++v) {
    const int u = v * kPwThreads + tid;
    const int i = u >> 5;
    const long p = pc + 8 * (u & 31);
    const bool ok = i < I && p < P;
    const pw_u32x4 t = *reinterpret_cast<const pw_u32x4 *>(xb + (ok ? (size_t)i * P + p : 0));
    r[v] = ok ? t : pw_u32x4{0u, 0u, 0u, 0u};
  }
}

template <int KB>
__device__ __forceinline__ void mixmx_put(uint16_t *xs, int tid, const pw_u32x4 (&r)[KB * 4]) {
#pragma unroll
  for (int v = 0; v < KB * 4; ++v) {
    const int u = v * kPwThreads + tid;
    uint2 *d = reinterpret_cast<uint2 *>(xs + (u >> 5) * kMxPitch + 8 * (u & 31));
    d[0] = make_uint2(r[v][0], r[v][1]);
    d[1] = make_uint2(r[v][2], r[v][3]);
  }
}

template <int DT>
__device__ __forceinline__ void load4h(const void *p, size_t i, float (&v)[4]) {
  const uint2 q = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(p) + i);
  if constexpr (DT == DT_F16) {
    const half2_t h0 = __builtin_bit_cast(half2_t, q.x), h1 = __builtin_bit_cast(half2_t, q.y);
    v[0] = (float)h0.x; v[1] = (float)h0.y; v[2] = (float)h1.x; v[3] = (float)h1.y;
  } else {
    v[0] = __uint_as_float(q.x << 16); v[1] = __uint_as_float(q.x & 0xffff0000u);
    v[2] = __uint_as_float(q.y << 16); v[3] = __uint_as_float(q.y & 0xffff0000u);
  }
}

// eight consecutive storage halves -> fp32
template <int DT>
__device__ __forceinline__ void unpack8(pw_u32x4 q, float (&v)[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if constexpr (DT == DT_F16) {
      // each half converted on its own: converting both lanes of a bit-cast
      // half2 taken from this vector gave wrong values for all but its first
      // element on gfx950
      v[2 * k] = (float)__builtin_bit_cast(_Float16, (uint16_t)(q[k] & 0xffffu));
      v[2 * k + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(q[k] >> 16));
    } else {
      v[2 * k] = __uint_as_float(q[k] << 16);
      v[2 * k + 1] = __uint_as_float(q[k] & 0xffff0000u);
    }
  }
}

template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (DT == DT_F16) {
    half2_t h;
    h.x = (_Float16)lo;
    h.y = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, h);
  } else {
    return f32x2_to_bf16x2(lo, hi);
  }
}

constexpr int kYsPitch = kMxPx + 1;  // floats per row of the output stage: the 16 rows x 4 pixel
                                     // groups one accumulator write touches fall on 64 distinct banks
constexpr int kYsRows = 32;          // output channels staged at a time

template <int DT, int KB>
__global__ __launch_bounds__(kPwThreads) __attribute__((amdgpu_waves_per_eu(2))) void fno_channel_mix_mx(MixArgs a) {
  constexpr int XS = KB * 32 * kMxPitch * 2, YS = kYsRows * kYsPitch * 4;
  __shared__ __attribute__((aligned(16))) unsigned char lds[XS > YS ? XS : YS];
  uint16_t *xs = reinterpret_cast<uint16_t *>(lds);
  float *ys = reinterpret_cast<float *>(lds);  // reused after the products
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int o0 = blockIdx.y * kOB, b = blockIdx.z;
  const int I = a.I, O = a.O;
  const long P = a.P;
  const uint16_t *xb = reinterpret_cast<const uint16_t *>(a.x) + (size_t)b * I * P;
  const size_t yb = (size_t)b * O * P;

  // B fragments: lane l holds W[o0 + 16 ot + l % 16][32 kb + 8 (l / 16) + t], t = 0..7
  pw_u32x4 wf[4][KB];
  const uint16_t *A = reinterpret_cast<const uint16_t *>(a.A);
#pragma unroll
  for (int ot = 0; ot < 4; ++ot)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int o = o0 + 16 * ot + (lane & 15);
      uint32_t h[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int i = 32 * kb + 8 * (lane >> 4) + t;
        h[t] = (o < O && i < I) ? A[(size_t)o * I + i] : 0u;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) wf[ot][kb][q] = h[2 * q] | (h[2 * q + 1] << 16);
    }
  float bias[4];
#pragma unroll
  for (int ot = 0; ot < 4; ++ot) {
    const int o = o0 + 16 * ot + (lane & 15);
    bias[ot] = (a.bias && o < O) ? load1<DT>(a.bias, o) : 0.f;
  }

  // Epilogue ownership: in staged half h (output channels o0 + 32 h ..
  // + 31), thread t handles row er = t / 8 and pixels 8 (t % 8) + 64 k,
  // k = 0..3: each 16-byte access of a wave covers 8 rows x 128 bytes.
  const int er = tid >> 3, ep = 8 * (tid & 7);
  // a contiguous run of tiles per workgroup, the next tile's channels in
  // flight while the current one is multiplied and written
  const long nch = (P + kMxPx - 1) / kMxPx, per = (nch + gridDim.x - 1) / gridDim.x;
  const long c0 = (long)blockIdx.x * per, c1 = min(nch, c0 + per);
  // the add input of the tile at pixel q (rows of this thread's epilogue)
  auto fetch_add = [&](long q, pw_u32x4 (&ad)[2][4]) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int o = o0 + 32 * h + er;
        const long p = q + ep + 64 * k;
        const bool ok = a.add && o < O && p < P;  // P % 8 == 0: 8 pixels wholly in or out
        const pw_u32x4 t = *reinterpret_cast<const pw_u32x4 *>(
            reinterpret_cast<const uint16_t *>(a.add ? a.add : a.x) + (ok ? yb + (size_t)o * P + p : 0));
        ad[h][k] = ok ? t : pw_u32x4{0u, 0u, 0u, 0u};
      }
  };
  pw_u32x4 r[KB * 4];
  long pc = c0 * kMxPx;
  if (c0 < c1) mixmx_fetch<KB>(xb, I, P, pc, tid, r);
  for (long c = c0; c < c1; ++c, pc += kMxPx) {
    mixmx_put<KB>(xs, tid, r);
    __syncthreads();
    pw_u32x4 ad[2][4];  // this tile's add input, in flight during the products
    fetch_add(pc, ad);
    if (c + 1 < c1) mixmx_fetch<KB>(xb, I, P, pc + kMxPx, tid, r);
    // Row r of product tile pt is pixel 64 wv + 4 r + pt: lane l's
    // accumulator j of tile pt is pixel 64 wv + 16 (l / 16) + 4 j + pt of
    // output channel 16 ot + l % 16.
    v4f acc[4][4];  // [pt][ot]
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      // A fragments: pixel 64 wv + 4 (l % 16) + pt, channels 32 kb + 8 (l / 16) .. + 7
      const uint16_t *col = xs + (8 * (lane >> 4)) * kMxPitch + 64 * wv + 4 * (lane & 15) + pt;
      pw_u32x4 af[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          af[kb][q] = (uint32_t)col[(32 * kb + 2 * q) * kMxPitch] | ((uint32_t)col[(32 * kb + 2 * q + 1) * kMxPitch] << 16);
#pragma unroll
      for (int ot = 0; ot < 4; ++ot) {
        acc[pt][ot] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) acc[pt][ot] = pw_mma<DT>(af[kb], wf[ot][kb], acc[pt][ot]);
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      __syncthreads();  // the channel tile (h = 0) or the previous half (h = 1) is no longer read
#pragma unroll
      for (int oq = 0; oq < 2; ++oq) {
        const int ot = 2 * h + oq;
        float *row = ys + (16 * oq + (lane & 15)) * kYsPitch + 64 * wv + 16 * (lane >> 4);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
          for (int j = 0; j < 4; ++j) row[4 * j + pt] = acc[pt][ot][j] + bias[ot];
      }
      __syncthreads();
      const int o = o0 + 32 * h + er;
      if (o < O) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const long p = pc + ep + 64 * k;
          if (p >= P) continue;
          const float *src = ys + er * kYsPitch + ep + 64 * k;
          float v[8];
          unpack8<DT>(ad[h][k], v);
          pw_u32x4 out;
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            float t0 = v[e] + src[e], t1 = v[e + 1] + src[e + 1];
            if (a.act == 1) {
              t0 = gelu_half(t0);
              t1 = gelu_half(t1);
            }
            out[e >> 1] = pack2<DT>(t0, t1);
          }
          *reinterpret_cast<pw_u32x4 *>(reinterpret_cast<uint16_t *>(a.y) + yb + (size_t)o * P + p) = out;
        }
      }
    }
    __syncthreads();
  }
}

// ----------------------------- FNO block: inverse row stage + 1x1 + act
//
// One block of the FNO module, y = act(K x + Wb x + b) (TurboFNO write-up,
// sections 1 and 4.3: the spectral layer sits inside such blocks), with the
// spectral convolution K finished here: the inverse plane kernel's column
// stage leaves the scaled fp16 rows of Z = E' Y ([B][H][Co][32 NN] halves,
// one power-of-two exponent per plane), and this kernel applies the row
// stage y = Z T' per image row and adds the 1x1 convolution in the same
// matrix-core accumulators. With M = 16 pixels of the row and N = 16 output
// channels, lane l holds channel o = l % 16 of pixels 4 (l / 16) .. + 3 in
// both products: the row-stage sum is unscaled in place (one exponent per
// lane) and the bypass products are added to the same registers; bias and
// act follow, and the block output is the only store. The spectral branch's
// output never leaves the chip.
//
// Workgroups are persistent: workgroup g takes rows g, g + G, ... of the
// B H (batch, row) pairs for its block of 64 output channels, keeping the
// T' and Wb fragments in registers for all of them. W / 64 waves, wave w
// owns pixels 64 w .. 64 w + 63 (four 16-pixel tiles). A row of x (32 KC
// channels, zero past Ci) goes through LDS [ci][px] (pitch W + 4 halves, two
// buffers) for the bypass's A fragments; the Z fragments come straight from
// global memory (64-byte pieces of Z rows). The next row's x and Z are
// requested before the current row's bypass products and epilogue, so
// they are in flight while those run; one barrier per row.
struct BlockRowArgs {
  const uint16_t *zg;       // [B][H][Co][32 NN] fp16 (re, im) pairs of Z, scaled
  const signed char *zexp;  // [B][Co]: Z = stored Z * 2^-zexp
  const pw_u32x4 *tb;       // T' fragments (A operand) [W / 16][NN][64 lanes]
  const void *x;            // [B][Ci][H][W]
  const void *wb;           // [Co][Ci]
  const void *bias;         // [Co] or null
  void *y;                  // [B][Co][H][W]
  int B, Ci, Co, H, NN, act;
};

template <int W, int KC>
__device__ __forceinline__ void brow_fetch_x(const BlockRowArgs &a, int row, int tid,
                                             pw_u32x4 (&xr)[KC * 32 * (W / 8) / W]) {
  constexpr int NT = W, XU = KC * 32 * (W / 8) / NT;
  const uint16_t *xb = reinterpret_cast<const uint16_t *>(a.x);
  const int b = row / a.H, h = row - b * a.H;
#pragma unroll
  for (int v = 0; v < XU; ++v) {
    const int u = v * NT + tid, ci = u / (W / 8), c = u % (W / 8);
    const bool ok = ci < a.Ci;
    const pw_u32x4 t =
        *reinterpret_cast<const pw_u32x4 *>(xb + (ok ? (((size_t)b * a.Ci + ci) * a.H + h) * W + 8 * c : 0));
    xr[v] = ok ? t : pw_u32x4{0u, 0u, 0u, 0u};
  }
}

// Z fragments of one row (B operand of the row stage: n = output channel,
// k = 8 halves of its Z row) and the planes' scales
__device__ __forceinline__ void brow_fetch_z(const BlockRowArgs &a, int row, int o0, int lane, pw_u32x4 (&zf)[4][2],
                                             int (&ze)[4]) {
  const int b = row / a.H, NN = a.NN, Co = a.Co;
#pragma unroll
  for (int ot = 0; ot < 4; ++ot) {
    const int o = o0 + 16 * ot + (lane & 15), oc = min(o, Co - 1);
    const uint16_t *zr = a.zg + ((size_t)row * Co + oc) * 32 * NN + 8 * (lane >> 4);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const pw_u32x4 t = *reinterpret_cast<const pw_u32x4 *>(zr + 32 * min(kb, NN - 1));
      zf[ot][kb] = (o < Co && kb < NN) ? t : pw_u32x4{0u, 0u, 0u, 0u};
    }
    ze[ot] = a.zexp[(size_t)b * Co + oc];
  }
}

template <int DT, int NW, int KC>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void fno_block_rows(BlockRowArgs a) {
  constexpr int W = NW * 64, XP = W + 4, NT = NW * 64;
  constexpr int XU = KC * 32 * (W / 8) / NT;  // 16-byte units of an x row per thread
  constexpr int XB = KC * 32 * XP;            // halves per LDS row buffer
  __shared__ __attribute__((aligned(16))) uint16_t xs[2 * XB];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int o0 = blockIdx.y * 64;
  const int Ci = a.Ci, Co = a.Co, H = a.H, NN = a.NN;
  const int rows = a.B * H;
  int row = blockIdx.x;
  if (row >= rows) return;

  // the first row's x and Z are requested before the fragments below
  pw_u32x4 xr[XU], zf[4][2];
  int ze[4];
  brow_fetch_x<W, KC>(a, row, tid, xr);
  brow_fetch_z(a, row, o0, lane, zf, ze);

  // T' fragments of the wave's four pixel tiles
  pw_u32x4 tf[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const pw_u32x4 t = a.tb[((size_t)(4 * wv + i) * NN + min(kb, NN - 1)) * 64 + lane];
      tf[i][kb] = kb < NN ? t : pw_u32x4{0u, 0u, 0u, 0u};
    }
  // Wb fragments (B operand of the bypass: n = output channel, k = input
  // channels 32 kc + 8 (l / 16) .. + 7; one 16-byte load where Ci allows)
  // and the bias
  pw_u32x4 wf[4][KC];
  float bias[4];
  const uint16_t *wb = reinterpret_cast<const uint16_t *>(a.wb);
  const bool wvec = (Ci & 7) == 0 && (reinterpret_cast<uintptr_t>(a.wb) & 15) == 0;
#pragma unroll
  for (int ot = 0; ot < 4; ++ot) {
    const int o = o0 + 16 * ot + (lane & 15);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int c0 = 32 * kc + 8 * (lane >> 4);
      if (wvec) {
        const bool ok = o < Co && c0 < Ci;
        const pw_u32x4 t = *reinterpret_cast<const pw_u32x4 *>(wb + (ok ? (size_t)o * Ci + c0 : 0));
        wf[ot][kc] = ok ? t : pw_u32x4{0u, 0u, 0u, 0u};
      } else {
        uint32_t hv[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const bool ok = o < Co && c0 + t < Ci;
          const uint32_t v = wb[ok ? (size_t)o * Ci + c0 + t : 0];
          hv[t] = ok ? v : 0u;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) wf[ot][kc][q] = hv[2 * q] | (hv[2 * q + 1] << 16);
      }
    }
    bias[ot] = (a.bias && o < Co) ? load1<DT>(a.bias, o) : 0.f;
  }

  for (int it = 0; row < rows; ++it, row += gridDim.x) {
    uint16_t *xsb = xs + (it & 1) * XB;
    // this row's x into its LDS buffer (the buffer's previous row was read
    // before the last barrier)
#pragma unroll
    for (int v = 0; v < XU; ++v) {
      const int u = v * NT + tid, ci = u / (W / 8), c = u % (W / 8);
      uint2 *d = reinterpret_cast<uint2 *>(xsb + ci * XP + 8 * c);
      d[0] = make_uint2(xr[v][0], xr[v][1]);
      d[1] = make_uint2(xr[v][2], xr[v][3]);
    }
    // row stage: acc[ot][i] = channel o0 + 16 ot + l % 16 at pixels
    // 64 wv + 16 i + 4 (l / 16) + j, unscaled per lane
    v4f acc[4][4];
#pragma unroll
    for (int ot = 0; ot < 4; ++ot) {
      const float isc = pow2f(-ze[ot]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v4f c = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          if (kb < NN) c = pw_mma<DT_F16>(tf[i][kb], zf[ot][kb], c);
        acc[ot][i] = c * isc;
      }
    }
    const int b = row / H, h = row - b * H;
    // the next row's x and Z are requested now (past the last row: this one
    // again, unused)
    const int nrow = row + (int)gridDim.x < rows ? row + (int)gridDim.x : row;
    brow_fetch_x<W, KC>(a, nrow, tid, xr);
    brow_fetch_z(a, nrow, o0, lane, zf, ze);
    __syncthreads();

    // bypass: A fragments of 16 pixels x 32 input channels from the row
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const uint16_t *col = xsb + (32 * kc + 8 * (lane >> 4)) * XP + 64 * wv + 16 * i + (lane & 15);
        pw_u32x4 af;
#pragma unroll
        for (int q = 0; q < 4; ++q) af[q] = (uint32_t)col[2 * q * XP] | ((uint32_t)col[(2 * q + 1) * XP] << 16);
#pragma unroll
        for (int ot = 0; ot < 4; ++ot) acc[ot][i] = pw_mma<DT>(af, wf[ot][kc], acc[ot][i]);
      }

    // bias, act, one 8-byte store of four pixels per (channel, tile)
#pragma unroll
    for (int ot = 0; ot < 4; ++ot) {
      const int o = o0 + 16 * ot + (lane & 15);
      if (o < Co) {
        uint16_t *yr =
            reinterpret_cast<uint16_t *>(a.y) + (((size_t)b * Co + o) * H + h) * W + 64 * wv + 4 * (lane >> 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            v[j] = acc[ot][i][j] + bias[ot];
            if (a.act == 1) v[j] = gelu_half(v[j]);
          }
          *reinterpret_cast<uint2 *>(yr + 16 * i) = make_uint2(pack2<DT>(v[0], v[1]), pack2<DT>(v[2], v[3]));
        }
      }
    }
  }
}

static constexpr int kMaxJ = 128;
static constexpr int kMaxC = 4;

template <int DT, bool AL>
__global__ __launch_bounds__(kPwThreads) void fno_projection(ProjArgs a) {
  __shared__ float q1w[kMaxJ * 64];  // [J][Ipad], Ipad <= 64
  __shared__ float q1b[kMaxJ];
  __shared__ float q2w[kMaxC * kMaxJ];
  __shared__ float q2b[kMaxC];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int b = blockIdx.z;
  const int I = a.I, J = a.J, C = a.C;
  const long P = a.P;
  const int Ipad = (I + 3) & ~3;
  for (int v = threadIdx.x; v < kMaxJ * Ipad; v += kPwThreads) {
    const int j = v / Ipad, i = v - j * Ipad;
    q1w[v] = (j < J && i < I) ? load1<DT>(a.Q1, (size_t)j * I + i) : 0.f;
  }
  for (int v = threadIdx.x; v < kMaxJ; v += kPwThreads) q1b[v] = v < J ? load1<DT>(a.q1, v) : 0.f;
  for (int v = threadIdx.x; v < kMaxC * kMaxJ; v += kPwThreads) {
    const int c = v / kMaxJ, j = v - c * kMaxJ;
    q2w[v] = (c < C && j < J) ? load1<DT>(a.Q2, (size_t)c * J + j) : 0.f;
  }
  for (int v = threadIdx.x; v < kMaxC; v += kPwThreads) q2b[v] = v < C ? load1<DT>(a.q2, v) : 0.f;
  __syncthreads();

  const int kr = lane >> 4, n = lane & 15;
  const size_t xb = (size_t)b * I * P, yb = (size_t)b * C * P;
  const long ntiles = (P + 63) / 64;
  for (long tile = (long)blockIdx.x * 4 + wv; tile < ntiles; tile += (long)gridDim.x * 4) {
    const long p0 = tile * 64 + 4 * n;
    const int np = (int)min((long)4, max(0L, P - p0));
    float part[kMaxC][4];
    // the whole input column (I <= 64 channels: 16 steps of 4) is fetched
    // once per tile, before the first MFMA, and reused by both hidden chunks
    float xs[16][4];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int i = 4 * k + kr;
      load4<DT, AL>(a.x, xb + (size_t)(i < I ? i : 0) * P, p0, P, i < I, xs[k]);
    }
#pragma unroll
    for (int c = 0; c < kMaxC; ++c)
#pragma unroll
      for (int t = 0; t < 4; ++t) part[c][t] = 0.f;
    for (int jc = 0; jc < kMaxJ; jc += 64) {  // hidden units in chunks of 64
      v4f acc[4][4];
#pragma unroll
      for (int mo = 0; mo < 4; ++mo)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[mo][t] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if (4 * k >= Ipad) break;
        const int i = 4 * k + kr;
#pragma unroll
        for (int mo = 0; mo < 4; ++mo) {
          const float av = q1w[(jc + 16 * mo + n) * Ipad + i];
#pragma unroll
          for (int t = 0; t < 4; ++t)
            acc[mo][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, xs[k][t], acc[mo][t], 0, 0, 0);
        }
      }
#pragma unroll
      for (int mo = 0; mo < 4; ++mo)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int j = jc + 16 * mo + 4 * kr + jj;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float h = gelu(acc[mo][t][jj] + q1b[j]);
#pragma unroll
            for (int c = 0; c < kMaxC; ++c) part[c][t] = fmaf(q2w[c * kMaxJ + j], h, part[c][t]);
          }
        }
    }
    // sum the four row groups (lanes n, n+16, n+32, n+48) in a fixed order
#pragma unroll
    for (int c = 0; c < kMaxC; ++c)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float v0 = __shfl(part[c][t], n, 64), v1 = __shfl(part[c][t], n + 16, 64);
        const float v2 = __shfl(part[c][t], n + 32, 64), v3 = __shfl(part[c][t], n + 48, 64);
        part[c][t] = ((v0 + v1) + (v2 + v3)) + q2b[c];
      }
    if (kr == 0 && np > 0) {
      for (int c = 0; c < C; ++c) {
        float v[4] = {part[c][0], part[c][1], part[c][2], part[c][3]};
        store4<DT>(a.y, yb + (size_t)c * P + p0, np, AL, v);
      }
    }
  }
}

// ------------------------------------------- half-precision projection
//
// fp16 / bf16 storage, I <= 64, J <= 128, C <= 4: the first layer
// h = GELU(Q1 x + q1) on v_mfma_f32_16x16x32_{f16,bf16} exactly as the
// channel mix (LDS-staged channel tiles, contiguous runs of 256-pixel tiles
// per workgroup, D[p][j] with each lane holding 16 consecutive pixels of one
// hidden unit), in four passes of 32 hidden units. The second layer is per
// lane: for every pixel, Q2[c][j] h[j] of the lane's hidden units, then a
// reduce-scatter over the 16 lanes of a row group in four DPP steps (a fixed
// order), after which lane e of the group holds the full sum of pixel e. Outputs are stored per row as 64 consecutive pixels
// per wave.

// One step of the 16-lane reduce-scatter: lanes whose bit log2(M) is set keep
// values M .. 2M - 1, the others 0 .. M - 1, and add the partner's copy of
// the kept half. Partners by DPP within a row of 16 lanes: M = 8 row_ror:8
// (lane ^ 8), M = 4 row_half_mirror (lane ^ 7: bit 2 differs, bit 3 kept),
// M = 2 and 1 quad permutes (lane ^ 2, lane ^ 1). Over the four steps each
// lane's partners span all 16 lanes of its row.
template <int M>
__device__ __forceinline__ void rs_step(float (&v)[16], int lane) {
  constexpr int ctrl = M == 8 ? 0x128 : M == 4 ? 0x141 : M == 2 ? 0x4e : 0xb1;
  const bool up = lane & M;
#pragma unroll
  for (int k = 0; k < M; ++k) {
    const float keep = up ? v[k + M] : v[k], send = up ? v[k] : v[k + M];
    const float got = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(send), ctrl, 0xf, 0xf, true));
    v[k] = keep + got;
  }
}

template <int DT, int KB>
__global__ __launch_bounds__(kPwThreads) __attribute__((amdgpu_waves_per_eu(2))) void fno_projection_mx(ProjArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[KB * 32 * kMxPitch];
  __shared__ pw_u32x4 wfs[8][KB][64];  // B fragments of Q1, read per use
  __shared__ float q1s[kMaxJ], q2s[kMaxC][kMaxJ], q2b[kMaxC];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int b = blockIdx.z;
  const int I = a.I, J = a.J, C = a.C;
  const long P = a.P;
  const uint16_t *xb = reinterpret_cast<const uint16_t *>(a.x) + (size_t)b * I * P;
  const size_t yb = (size_t)b * C * P;
  for (int v = tid; v < kMaxJ; v += kPwThreads) q1s[v] = v < J ? load1<DT>(a.q1, v) : 0.f;
  for (int v = tid; v < kMaxC * kMaxJ; v += kPwThreads) {
    const int c = v / kMaxJ, j = v - c * kMaxJ;
    q2s[c][j] = (c < C && j < J) ? load1<DT>(a.Q2, (size_t)c * J + j) : 0.f;
  }
  if (tid < kMaxC) q2b[tid] = tid < C ? load1<DT>(a.q2, tid) : 0.f;

  // B fragments of Q1: lane l holds Q1[16 jt + l % 16][32 kb + 8 (l / 16) + t];
  // wave w builds those of jt = 2 w, 2 w + 1
  const uint16_t *Q1 = reinterpret_cast<const uint16_t *>(a.Q1);
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int jt = 2 * wv + jj, j = 16 * jt + (lane & 15);
      uint32_t h[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int i = 32 * kb + 8 * (lane >> 4) + t;
        h[t] = (j < J && i < I) ? Q1[(size_t)j * I + i] : 0u;
      }
      pw_u32x4 f;
#pragma unroll
      for (int q = 0; q < 4; ++q) f[q] = h[2 * q] | (h[2 * q + 1] << 16);
      wfs[jt][kb][lane] = f;
    }

  const long nch = (P + kMxPx - 1) / kMxPx, per = (nch + gridDim.x - 1) / gridDim.x;
  const long c0 = (long)blockIdx.x * per, c1 = min(nch, c0 + per);
  pw_u32x4 r[KB * 4];
  long pc = c0 * kMxPx;
  if (c0 < c1) mixmx_fetch<KB>(xb, I, P, pc, tid, r);
  for (long c = c0; c < c1; ++c, pc += kMxPx) {
    mixmx_put<KB>(xs, tid, r);
    __syncthreads();
    if (c + 1 < c1) mixmx_fetch<KB>(xb, I, P, pc + kMxPx, tid, r);
    float outv[kMaxC] = {0.f, 0.f, 0.f, 0.f};  // lane e of a row group: pixel e of the group
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {  // hidden units in passes of 32 (two 16-wide tiles)
      v4f acc[4][2];  // [pt][jt within the pass]
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        // A fragments: pixel 64 wv + 4 (l % 16) + pt, channels 32 kb + 8 (l / 16) .. + 7
        const uint16_t *col = xs + (8 * (lane >> 4)) * kMxPitch + 64 * wv + 4 * (lane & 15) + pt;
        pw_u32x4 af[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            af[kb][q] =
                (uint32_t)col[(32 * kb + 2 * q) * kMxPitch] | ((uint32_t)col[(32 * kb + 2 * q + 1) * kMxPitch] << 16);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          acc[pt][q] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) acc[pt][q] = pw_mma<DT>(af[kb], wfs[2 * hh + q][kb][lane], acc[pt][q]);
        }
      }
      // h = GELU(acc + q1) in place; accumulator j of tile pt is pixel 4 j + pt of the group
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float bq = q1s[16 * (2 * hh + q) + (lane & 15)];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[pt][q][j] = gelu_half(acc[pt][q][j] + bq);
      }
#pragma unroll
      for (int cc = 0; cc < kMaxC; ++cc) {
        if (cc >= C) break;
        float v[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] = 0.f;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const float w2 = q2s[cc][16 * (2 * hh + q) + (lane & 15)];
#pragma unroll
          for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int j = 0; j < 4; ++j) v[4 * j + pt] = fmaf(w2, acc[pt][q][j], v[4 * j + pt]);
        }
        // reduce-scatter over the 16 lanes (hidden units) of the row group
        rs_step<8>(v, lane);
        rs_step<4>(v, lane);
        rs_step<2>(v, lane);
        rs_step<1>(v, lane);
        outv[cc] += v[0];
      }
    }
    const long p = pc + 64 * wv + 16 * (lane >> 4) + (lane & 15);
    if (p < P) {
#pragma unroll
      for (int cc = 0; cc < kMaxC; ++cc) {
        if (cc >= C) break;
        const float y = outv[cc] + q2b[cc];
        if constexpr (DT == DT_F16) reinterpret_cast<_Float16 *>(a.y)[yb + (size_t)cc * P + p] = (_Float16)y;
        else reinterpret_cast<uint16_t *>(a.y)[yb + (size_t)cc * P + p] = (uint16_t)f32_to_bf16(y);
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- launchers

static int pw_blocks(long P) {
  const long tiles = (P + 63) / 64;
  long blocks = (tiles + 3) / 4;
  return (int)(blocks < 4096 ? blocks : 4096);
}

// ------------------------------------------------ lift folded into block 0
//
// The lift v0 = P f + p (P [C][J], p [C], f the J feature channels) and the
// first block are linear in v0, so the first block can run on f directly:
//   spectral branch  Yh[b][o][k] = sum_j Xh_f[b][j][k] Wf[k][j][o]
//                    + (k = DC) sum_c p[c] w[0][c][o],
//     Wf[k][j][o] = sum_c P[c][j] w[k][c][o]  (the spectra of the constant
//     field p[c] are p[c] at the DC mode only, which the inverse turns into
//     the constant Re(sum_c p[c] w[0][c][o]) on every pixel);
//   bypass           sum_c Wb[o][c] v0[c] + b[o] = sum_j Af[o][j] f[j] + bf[o],
//     Af[o][j] = sum_c Wb[o][c] P[c][j],
//     bf[o] = sum_c Wb[o][c] p[c] + b[o] + Re(sum_c p[c] w[0][c][o]).
// Threads take (k, o) pairs, consecutive o on consecutive lanes (the weight
// rows w[k][c][0 .. C) are read coalesced, once for all J outputs of the
// pair, in chunks of four j); the last C threads form Af and bf. fp32 sums
// over c, rounded to the storage dtype. v0 itself is never formed.
struct FoldArgs {
  const void *P, *p, *w, *Wb, *b;  // P [C][J], p [C], w [K][C][C][2], Wb [C][C], b [C]
  void *wf, *af, *bf;              // wf [K][J][C][2], af [C][J], bf [C]
  int K, J, C;
};

template <int DT>
__device__ __forceinline__ void store1(void *p, size_t i, float v) {
  if constexpr (DT == DT_F32) reinterpret_cast<float *>(p)[i] = v;
  else if constexpr (DT == DT_F16) reinterpret_cast<_Float16 *>(p)[i] = (_Float16)v;
  else reinterpret_cast<uint16_t *>(p)[i] = (uint16_t)f32_to_bf16(v);
}

constexpr int kFoldP = kProjMaxIn * kMixMaxIn;  // P entries staged in LDS (C <= 64, J <= 128)

template <int DT>
__global__ __launch_bounds__(kPwThreads) void fno_lift_fold(FoldArgs a) {
  __shared__ float ps[kFoldP];  // P [C][J], fp32
  const int K = a.K, J = a.J, C = a.C;
  for (int v = threadIdx.x; v < C * J; v += kPwThreads) ps[v] = load1<DT>(a.P, v);
  __syncthreads();
  const long npair = (long)K * C, total = npair + C;
  for (long t = (long)blockIdx.x * kPwThreads + threadIdx.x; t < total; t += (long)gridDim.x * kPwThreads) {
    if (t < npair) {
      const int o = (int)(t % C);
      const long k = t / C;
      for (int j0 = 0; j0 < J; j0 += 4) {
        float re[4] = {0.f, 0.f, 0.f, 0.f}, im[4] = {0.f, 0.f, 0.f, 0.f};
        // the weights of 16 input channels are requested together (their
        // latencies overlap), clamped in range; past C they count as zero
        for (int c0 = 0; c0 < C; c0 += 16) {
          float2 wv[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) wv[u] = load_pair<DT>(a.w, ((size_t)(k * C + min(c0 + u, C - 1)) * C + o) * 2);
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            const int c = c0 + u;
            if (c < C) {
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const float pc = j0 + q < J ? ps[c * J + j0 + q] : 0.f;
                re[q] = fmaf(pc, wv[u].x, re[q]);
                im[q] = fmaf(pc, wv[u].y, im[q]);
              }
            }
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (j0 + q < J) store_pair<DT>(a.wf, (((size_t)k * J + j0 + q) * C + o) * 2, re[q], im[q]);
      }
    } else {
      // output channel o: row o of Af and bf[o]
      const int o = (int)(t - npair);
      float s = load1<DT>(a.b, o);
      for (int j0 = 0; j0 < J; j0 += 4) {
        float af[4] = {0.f, 0.f, 0.f, 0.f};
        for (int c0 = 0; c0 < C; c0 += 16) {
          float wb[16], pc[16], w0[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            const int c = min(c0 + u, C - 1);
            wb[u] = load1<DT>(a.Wb, (size_t)o * C + c);
            pc[u] = load1<DT>(a.p, c);
            w0[u] = load_pair<DT>(a.w, ((size_t)c * C + o) * 2).x;
          }
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            const int c = c0 + u;
            if (c < C) {
#pragma unroll
              for (int q = 0; q < 4; ++q) af[q] = fmaf(wb[u], j0 + q < J ? ps[c * J + j0 + q] : 0.f, af[q]);
              if (j0 == 0) s = fmaf(pc[u], wb[u] + w0[u], s);
            }
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (j0 + q < J) store1<DT>(a.af, (size_t)o * J + j0 + q, af[q]);
      }
      store1<DT>(a.bf, o, s);
    }
  }
}

hipError_t launch_lift_fold(const void *P, const void *p, const void *w, const void *Wb, const void *b, void *wf,
                            void *af, void *bf, int K, int J, int C, int dtype, hipStream_t s) {
  if (C * J > kFoldP) return hipErrorInvalidValue;
  FNO_BOUNDS(check_lift_fold(P, p, w, Wb, b, wf, af, bf, K, J, C, dtype);)
  FoldArgs a{P, p, w, Wb, b, wf, af, bf, K, J, C};
  void *args[] = {(void *)&a};
  const long total = (long)K * C + C;
  const unsigned g = (unsigned)std::min<long>((total + kPwThreads - 1) / kPwThreads, 4096);
  const void *k = dtype == DT_F32 ? (const void *)fno_lift_fold<DT_F32>
                  : dtype == DT_F16 ? (const void *)fno_lift_fold<DT_F16>
                                    : (const void *)fno_lift_fold<DT_BF16>;
  return hipLaunchKernel(k, dim3(g), dim3(kPwThreads), args, 0, s);
}

hipError_t launch_channel_mix(const void *x, const void *A, const void *bias, const void *add, void *y, int B,
                              int I, int O, long P, int act, int dtype, hipStream_t s) {
  FNO_BOUNDS(check_channel_mix(x, A, bias, add, y, B, I, O, P, dtype);)
  MixArgs a{x, A, bias, add, y, B, I, O, P, act};
  void *args[] = {(void *)&a};
  if (dtype != DT_F32 && (P & 7) == 0 && I <= 64) {
    const int KB = I <= 32 ? 1 : 2;
    // about 1024 workgroups in all (four per CU), each a contiguous run of tiles
    const long nch = (P + kMxPx - 1) / kMxPx, rest = (long)B * ((O + kOB - 1) / kOB);
    const long gx = std::min(nch, std::max(1L, (1024 + rest - 1) / rest));
    dim3 g((unsigned)gx, (O + kOB - 1) / kOB, B);
    const void *k = dtype == DT_F16 ? (KB == 1 ? (const void *)fno_channel_mix_mx<DT_F16, 1>
                                               : (const void *)fno_channel_mix_mx<DT_F16, 2>)
                                    : (KB == 1 ? (const void *)fno_channel_mix_mx<DT_BF16, 1>
                                               : (const void *)fno_channel_mix_mx<DT_BF16, 2>);
    return hipLaunchKernel(k, g, dim3(kPwThreads), args, 0, s);
  }
  dim3 grid(pw_blocks(P), (O + kOB - 1) / kOB, B);
  const bool al = (P & 3) == 0;
  const void *k = dtype == DT_F32 ? (al ? (const void *)fno_channel_mix<DT_F32, true>
                                        : (const void *)fno_channel_mix<DT_F32, false>)
                  : dtype == DT_F16 ? (al ? (const void *)fno_channel_mix<DT_F16, true>
                                          : (const void *)fno_channel_mix<DT_F16, false>)
                                    : (al ? (const void *)fno_channel_mix<DT_BF16, true>
                                          : (const void *)fno_channel_mix<DT_BF16, false>);
  return hipLaunchKernel(k, grid, dim3(kPwThreads), args, 0, s);
}

hipError_t launch_projection(const void *x, const void *Q1, const void *q1, const void *Q2, const void *q2, void *y,
                             int B, int I, int J, int C, long P, int dtype, hipStream_t s) {
  FNO_BOUNDS(check_projection(x, Q1, q1, Q2, q2, y, B, I, J, C, P, dtype);)
  ProjArgs a{x, Q1, q1, Q2, q2, y, B, I, J, C, P};
  void *args[] = {(void *)&a};
  if (dtype != DT_F32 && (P & 7) == 0 && I <= 64 && J <= kMaxJ && C <= kMaxC) {
    const int KB = I <= 32 ? 1 : 2;
    const long nch = (P + kMxPx - 1) / kMxPx;
    const long gx = std::min(nch, std::max(1L, (1024L + B - 1) / B));
    const void *k = dtype == DT_F16 ? (KB == 1 ? (const void *)fno_projection_mx<DT_F16, 1>
                                               : (const void *)fno_projection_mx<DT_F16, 2>)
                                    : (KB == 1 ? (const void *)fno_projection_mx<DT_BF16, 1>
                                               : (const void *)fno_projection_mx<DT_BF16, 2>);
    return hipLaunchKernel(k, dim3((unsigned)gx, 1, B), dim3(kPwThreads), args, 0, s);
  }
  dim3 grid(pw_blocks(P), 1, B);
  const bool al = (P & 3) == 0;
  const void *k = dtype == DT_F32 ? (al ? (const void *)fno_projection<DT_F32, true>
                                        : (const void *)fno_projection<DT_F32, false>)
                  : dtype == DT_F16 ? (al ? (const void *)fno_projection<DT_F16, true>
                                          : (const void *)fno_projection<DT_F16, false>)
                                    : (al ? (const void *)fno_projection<DT_BF16, true>
                                          : (const void *)fno_projection<DT_BF16, false>);
  return hipLaunchKernel(k, grid, dim3(kPwThreads), args, 0, s);
}


template <int DT, int NW>
static const void *block_rows_kernel(int KC) {
  return KC == 1 ? (const void *)fno_block_rows<DT, NW, 1> : (const void *)fno_block_rows<DT, NW, 2>;
}

bool block_rows_supported(int dtype, int W, int Ci, int NN) {
  return (dtype == DT_F16 || dtype == DT_BF16) && (W == 64 || W == 128 || W == 256) && Ci >= 1 && Ci <= 64 &&
         (NN == 1 || NN == 2);
}

hipError_t launch_block_rows(const uint16_t *zg, const signed char *zexp, const void *tb, const void *x,
                             const void *wb, const void *bias, void *y, int B, int Ci, int Co, int H, int W, int NN,
                             int act, int dtype, hipStream_t s) {
  if (!block_rows_supported(dtype, W, Ci, NN) || B < 1 || B > 65535 || H < 1 || Co < 1) return hipErrorInvalidValue;
  FNO_BOUNDS(check_block_rows(zg, zexp, tb, x, wb, bias, y, B, Ci, Co, H, W, NN, dtype);)
  BlockRowArgs a{zg, zexp, reinterpret_cast<const pw_u32x4 *>(tb), x, wb, bias, y, B, Ci, Co, H, NN, act};
  void *args[] = {(void *)&a};
  const int KC = Ci <= 32 ? 1 : 2, NW = W / 64;
  const void *k = nullptr;
  if (dtype == DT_F16)
    k = NW == 1 ? block_rows_kernel<DT_F16, 1>(KC) : NW == 2 ? block_rows_kernel<DT_F16, 2>(KC) : block_rows_kernel<DT_F16, 4>(KC);
  else
    k = NW == 1 ? block_rows_kernel<DT_BF16, 1>(KC) : NW == 2 ? block_rows_kernel<DT_BF16, 2>(KC)
                                                   : block_rows_kernel<DT_BF16, 4>(KC);
  // persistent: about two workgroups per CU, rows dealt round-robin
  int dev = 0, ncu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const long rows = (long)B * H, nob = (Co + 63) / 64;
  if (rows > 0x7fffffffL) return hipErrorInvalidValue;
  const long g = std::max(1L, std::min(rows, (2L * ncu + nob - 1) / nob));
  return hipLaunchKernel(k, dim3((unsigned)g, (unsigned)nob), dim3(NW * 64), args, 0, s);
}

}  // namespace fno
