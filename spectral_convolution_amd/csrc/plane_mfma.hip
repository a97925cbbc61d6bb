// plane_mfma.hip - plane transforms for fp16 / bf16 storage whose row stage
// (the contiguous, real axis, which touches every input and output element)
// is a truncated DFT on matrix cores.
//
// The row stage of the layer only needs m2 << W outputs (forward) or inputs
// (inverse) per row: R[h][c] = sum_w x[h][w] T[w][c] with T[w][2ky] =
// cos(2 pi ky w / W), T[w][2ky+1] = -sin(2 pi ky w / W); and back,
// y[h][w] = sum_c Z'[h][c] T'[c][w] with T'[2ky][w] = g cos(2 pi ky w / W),
// T'[2ky+1][w] = -g sin(2 pi ky w / W), g = 1 for ky = 0 (which also drops
// Im Z[h][0]) and 2 otherwise. Both are dense [rows x W] x [W x 2 m2]
// contractions with fp32 accumulation: v_mfma_f32_16x16x32_{f16,bf16}.
// The twiddle matrices come from host tables already in MFMA fragment order.
// The column stages stay pruned FFT butterflies on the VALU in fp32
// (plane_common.hpp).
//
// Precision. Forward fp16: x is exact, T is rounded to fp16. Forward bf16:
// x is exact and T = T_hi + T_lo (two bf16 products), so inputs of any bf16
// magnitude are safe. Inverse (both dtypes): Z is scaled by a power of two
// chosen from the plane's max |Z| into fp16 range, T' rounded to fp16, and the
// fp32 result is unscaled before the final RNE rounding to the storage dtype.
//
// Layout of one fragment of v_mfma_f32_16x16x32 (A: 16 x 32, B: 32 x 16):
// lane l holds row / column l % 16 and the eight consecutive k = 8 (l / 16)
// .. 8 (l / 16) + 7; accumulator register j of lane l holds row 4 (l / 16) + j,
// column l % 16.

#include "plane_common.hpp"

namespace fno {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v4f mfma16(uint4 a, uint4 b, v4f c, bool bf) {
  if (bf)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, a), __builtin_bit_cast(b8, b), c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c, 0, 0, 0);
}

constexpr int kRound = 64; // rows staged per round (four 16-row stripes)

int mx_ntiles(int m2) { return m2 <= 8 ? 1 : m2 <= 16 ? 2 : 4; }

size_t mx_fwd_lds_bytes(int H, int W, int m2) {
  return ((size_t)H + (size_t)H * (m2 + 1)) * sizeof(float2) + (size_t)kRound * (W * 2 + 16);
}

size_t mx_inv_lds_bytes(int H, int W, int m1, int m2) {
  return ((size_t)H + (size_t)2 * m1 * m2 + (size_t)H * (m2 + 1)) * sizeof(float2) + (size_t)16 * (W * 2 + 16) + 64;
}

// in-flight row data uses a native vector type: arrays of the HIP uint4
// struct that are carried around the round loop are not kept in registers
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <int KB>
__device__ __forceinline__ void mx_fetch(const uint4 *xp, int r, int WU, int tid, u32x4 (&p)[KB]) {
  const u32x4 *src = reinterpret_cast<const u32x4 *>(xp) + (size_t)r * kRound * WU + tid;
#pragma unroll
  for (int v = 0; v < KB; ++v) p[v] = src[v * kThreads];
}

template <int KB>
__device__ __forceinline__ void mx_put(uint4 *stage, int pitch, int WU, int tid, const u32x4 (&p)[KB]) {
#pragma unroll
  for (int v = 0; v < KB; ++v) {
    const int e = v * kThreads + tid;
    const int row = e / WU, cu = e - row * WU;
    reinterpret_cast<u32x4 *>(stage)[row * pitch + cu] = p[v];
  }
}

// R[h][c] for the 64 staged rows of round r: 4 stripes x NT column tiles of
// 16 x 16, wave wv takes tasks wv, wv + 4, ...; ct is this lane's column
template <int DT, int NT, int KB>
__device__ __forceinline__ void mx_row_dft(const uint4 *stage, int pitch, const uint4 (&th)[KB],
                                           const uint4 (&tl)[DT == DT_BF16 ? KB : 1], float2 *R, int m2, int ct,
                                           int r, int wv, int lane) {
  constexpr bool BF = DT == DT_BF16;
  for (int task = wv; task < 4 * NT; task += 4) {
    const int stripe = task / NT;
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    const uint4 *ar = stage + (stripe * 16 + (lane & 15)) * pitch + (lane >> 4);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const uint4 av = ar[kb * 4];
      acc = mfma16(av, th[kb], acc, BF);
      if constexpr (BF) acc = mfma16(av, tl[kb], acc, BF);
    }
    if (ct < 2 * m2) {
      float *rf = reinterpret_cast<float *>(R) + ct;
      const int h0 = r * kRound + stripe * 16 + 4 * (lane >> 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) rf[(size_t)(h0 + j) * 2 * (m2 + 1)] = acc[j];
    }
  }
}

template <int MP, int DT, int NT, int KB>
__global__ __launch_bounds__(kThreads) void fno_fwd_plane_mx(PlaneMxFwdArgs a) {
  extern __shared__ float2 smem[];
  constexpr bool BF = DT == DT_BF16;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int H = a.H, W = a.W, m1 = a.m1, m2 = a.m2, PH = a.PH;
  const int m2p = m2 + 1, WU = W / 8;  // WU: 16-byte units per row (W = 32 KB)
  const int pitch = WU + 1;                          // staged row pitch in 16-byte units
  float2 *twh = smem;
  float2 *R = twh + H;                                            // [H][m2 + 1]
  uint4 *stage = reinterpret_cast<uint4 *>(R + (size_t)H * m2p);  // [64][pitch]
  for (int v = tid; v < H; v += kThreads) twh[v] = a.tw_h[v];

  const int plane = blockIdx.x;
  const uint4 *xp = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(a.x) + (size_t)plane * H * W);

  // twiddle fragments of this wave's 16-column tile, all K-blocks
  const int nt = wv % NT;
  uint4 th[KB], tl[BF ? KB : 1];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    th[kb] = a.tf[((size_t)nt * KB + kb) * 64 + lane];
    if constexpr (BF) tl[kb] = a.tf_lo[((size_t)nt * KB + kb) * 64 + lane];
  }

  // rounds of 64 rows: every thread moves KB 16-byte units per round; two
  // rounds are in flight in registers while a third is multiplied from LDS
  const int rounds = H / kRound;
  const int ct = nt * 16 + (lane & 15);
  u32x4 pa[KB], pb[KB];
  mx_fetch<KB>(xp, 0, WU, tid, pa);
  if (rounds > 1) mx_fetch<KB>(xp, 1, WU, tid, pb);
  for (int r = 0; r < rounds; r += 2) {
    mx_put<KB>(stage, pitch, WU, tid, pa);
    __syncthreads();
    if (r + 2 < rounds) mx_fetch<KB>(xp, r + 2, WU, tid, pa);
    mx_row_dft<DT, NT, KB>(stage, pitch, th, tl, R, m2, ct, r, wv, lane);
    __syncthreads();
    if (r + 1 < rounds) {
      mx_put<KB>(stage, pitch, WU, tid, pb);
      __syncthreads();
      if (r + 3 < rounds) mx_fetch<KB>(xp, r + 3, WU, tid, pb);
      mx_row_dft<DT, NT, KB>(stage, pitch, th, tl, R, m2, ct, r + 1, wv, lane);
      __syncthreads();
    }
  }

  // ---- column stage (VALU butterflies, fp32)
  fwd_col_stage<MP>(R, 1, plane, H, m1, m2, PH, a.rc, twh, a.out, a.scale);
}

template <int MP, int DT, int KBT>
__global__ __launch_bounds__(kThreads) void fno_inv_plane_mx(PlaneMxInvArgs a) {
  extern __shared__ float2 smem[];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int H = a.H, W = a.W, m1 = a.m1, m2 = a.m2, PH = a.PH;
  const int m2p = m2 + 1, K = 2 * m1 * m2, WU = W / 8, pitch = WU + 1;
  float2 *twh = smem;
  float2 *Yh = twh + H;                                                 // [K]
  float2 *Zb = Yh + K;                                                  // [H][m2 + 1]
  uint4 *ostage = reinterpret_cast<uint4 *>(Zb + (size_t)H * m2p);     // [16][pitch]
  unsigned *zmax = reinterpret_cast<unsigned *>(ostage + 16 * pitch);
  const int plane = blockIdx.x;
  for (int v = tid; v < H; v += kThreads) twh[v] = a.tw_h[v];
  for (int v = tid; v < K; v += kThreads) Yh[v] = a.in[(size_t)plane * K + v];
  if (tid == 0) *zmax = 0u;
  __syncthreads();

  inv_col_stage<MP>(Yh, Zb, 1, H, m1, m2, PH, twh);
  __syncthreads();

  // power-of-two scale that brings max |Z| to [2^13, 2^14): fp16 range for
  // the A operand, most of its precision for the largest values
  {
    float mx = 0.f;
    for (int v = tid; v < H * m2; v += kThreads) {
      const int h = v / m2, ky = v - h * m2;
      const float2 z = Zb[(size_t)h * m2p + ky];
      mx = fmaxf(mx, fmaxf(fabsf(z.x), fabsf(z.y)));
    }
    mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 4, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 8, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (lane == 0) atomicMax(zmax, __float_as_uint(mx));
  }
  __syncthreads();
  const float zm = __uint_as_float(*zmax);
  int ex = 0;
  if (zm > 0.f && zm < 3.0e38f) (void)frexpf(zm, &ex);  // zm in [2^(ex-1), 2^ex)
  const float sc = zm > 0.f ? ldexpf(1.f, 14 - ex) : 1.f;
  const float isc = zm > 0.f ? ldexpf(1.f, ex - 14) : 1.f;

  // this wave's output column tiles: wv, wv + 4, ... (W / 64 of them); the
  // inverse twiddle fragments for them stay in registers
  constexpr int kMaxWT = 4;
  const int nwt = W / 64;
  uint4 tb[kMaxWT][KBT];
#pragma unroll
  for (int i = 0; i < kMaxWT; ++i)
    if (i < nwt) {
      const int wt = wv + 4 * i;
#pragma unroll
      for (int kb = 0; kb < KBT; ++kb) tb[i][kb] = a.tb[((size_t)wt * KBT + kb) * 64 + lane];
    }

  const float *zf = reinterpret_cast<const float *>(Zb);
  const size_t ybase = (size_t)plane * H * W;
  for (int stripe = 0; stripe < H / 16; ++stripe) {
    // A fragments: Z rows of the stripe, c = 8 (l / 16) + i (+ 32 kb), scaled to fp16
    uint4 af[KBT];
    const int h = stripe * 16 + (lane & 15);
#pragma unroll
    for (int kb = 0; kb < KBT; ++kb) {
      half2_t hv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = kb * 32 + 8 * (lane >> 4) + 2 * i;
        float v0 = 0.f, v1 = 0.f;
        if (c < 2 * m2) {
          const float2 z = *reinterpret_cast<const float2 *>(zf + (size_t)h * 2 * m2p + c);
          v0 = z.x * sc;
          v1 = z.y * sc;
        }
        hv[i].x = (_Float16)v0;
        hv[i].y = (_Float16)v1;
      }
      af[kb] = make_uint4(__builtin_bit_cast(uint32_t, hv[0]), __builtin_bit_cast(uint32_t, hv[1]),
                          __builtin_bit_cast(uint32_t, hv[2]), __builtin_bit_cast(uint32_t, hv[3]));
    }
#pragma unroll
    for (int i = 0; i < kMaxWT; ++i) {
      if (i < nwt) {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KBT; ++kb) acc = mfma16(af[kb], tb[i][kb], acc, false);
        const int w = (wv + 4 * i) * 16 + (lane & 15);
        uint16_t *os = reinterpret_cast<uint16_t *>(ostage);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float v = acc[j] * isc;
          uint16_t bits;
          if constexpr (DT == DT_F16) bits = __builtin_bit_cast(uint16_t, (_Float16)v);
          else bits = (uint16_t)f32_to_bf16(v);
          os[(size_t)(4 * (lane >> 4) + j) * pitch * 8 + w] = bits;
        }
      }
    }
    __syncthreads();
    // 16 rows x W halves, coalesced 16-byte stores
    uint4 *yp = reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(a.y) + ybase + (size_t)stripe * 16 * W);
    for (int e = tid; e < 16 * WU; e += kThreads) {
      const int row = e / WU, cu = e - row * WU;
      yp[e] = ostage[row * pitch + cu];
    }
    __syncthreads();
  }
}

// --------------------------------------------------------------- launchers

template <int DT, int KB>
static const void *mx_fwd_kernel_kb(int MP, int nt) {
  switch (MP) {
    case 2: return (const void *)fno_fwd_plane_mx<2, DT, 1, KB>;
    case 4: return (const void *)fno_fwd_plane_mx<4, DT, 1, KB>;
    case 8: return (const void *)fno_fwd_plane_mx<8, DT, 1, KB>;
    case 16: return nt == 1 ? (const void *)fno_fwd_plane_mx<16, DT, 1, KB> : (const void *)fno_fwd_plane_mx<16, DT, 2, KB>;
    case 32:
      return nt == 1   ? (const void *)fno_fwd_plane_mx<32, DT, 1, KB>
             : nt == 2 ? (const void *)fno_fwd_plane_mx<32, DT, 2, KB>
                       : (const void *)fno_fwd_plane_mx<32, DT, 4, KB>;
  }
  return nullptr;
}

template <int DT>
static const void *mx_fwd_kernel(int MP, int nt, int W) {
  switch (W) {
    case 64: return mx_fwd_kernel_kb<DT, 2>(MP, nt);
    case 128: return mx_fwd_kernel_kb<DT, 4>(MP, nt);
    case 256: return mx_fwd_kernel_kb<DT, 8>(MP, nt);
  }
  return nullptr;
}

template <int DT>
static const void *mx_inv_kernel(int MP, int kbt) {
#define FNO_MXI(MPV) \
  case MPV:          \
    return kbt == 1 ? (const void *)fno_inv_plane_mx<MPV, DT, 1> : (const void *)fno_inv_plane_mx<MPV, DT, 2>;
  switch (MP) {
    FNO_MXI(2)
    FNO_MXI(4)
    FNO_MXI(8)
    FNO_MXI(16)
    FNO_MXI(32)
  }
#undef FNO_MXI
  return nullptr;
}

static const void *mx_kernel(bool fwd, int MP, int m2, int W, int dtype) {
  const int nt = mx_ntiles(m2), kbt = m2 <= 16 ? 1 : 2;
  if (nt > MP / 8 && nt > 1) return nullptr;  // m2 <= MP: tiles never exceed what MP allows
  if (dtype == DT_F16) return fwd ? mx_fwd_kernel<DT_F16>(MP, nt, W) : mx_inv_kernel<DT_F16>(MP, kbt);
  if (dtype == DT_BF16) return fwd ? mx_fwd_kernel<DT_BF16>(MP, nt, W) : mx_inv_kernel<DT_BF16>(MP, kbt);
  return nullptr;
}

bool mx_supported(int H, int W, int m2, int dtype) {
  return (dtype == DT_F16 || dtype == DT_BF16) && H >= kRound && W >= 64 && W <= 256 && m2 <= 32;
}

hipError_t mx_prepare(bool fwd, int MP, int m2, int W, int dtype, size_t lds) {
  const void *k = mx_kernel(fwd, MP, m2, W, dtype);
  if (!k) return hipErrorInvalidValue;
  return hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

hipError_t launch_plane_mx_fwd(const PlaneMxFwdArgs &a, int MP, int dtype, size_t lds, hipStream_t s) {
  const void *k = mx_kernel(true, MP, a.m2, a.W, dtype);
  if (!k) return hipErrorInvalidValue;
  void *args[] = {(void *)&a};
  return hipLaunchKernel(k, dim3(a.nplanes), dim3(kThreads), args, lds, s);
}

hipError_t launch_plane_mx_inv(const PlaneMxInvArgs &a, int MP, int dtype, size_t lds, hipStream_t s) {
  const void *k = mx_kernel(false, MP, a.m2, a.W, dtype);
  if (!k) return hipErrorInvalidValue;
  void *args[] = {(void *)&a};
  return hipLaunchKernel(k, dim3(a.nplanes), dim3(kThreads), args, lds, s);
}

}  // namespace fno
