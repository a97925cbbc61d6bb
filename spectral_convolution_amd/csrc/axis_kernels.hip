// axis_kernels.hip - pruned complex DFTs along a strided axis.
//
// Used for the outermost axis of a 3D layer (kx, two corners): the data is
// [vol][N][C] complex with C contiguous columns. A workgroup takes CT
// consecutive columns of one volume, so every load and store is coalesced
// along C. The decimation is the one the plane kernels use: residues r < P,
// MP-point register DFTs over n = r + P q, then (forward) a Horner combine
// over r in LDS, or (inverse) a per-residue pre-multiply of the retained
// inputs followed by one inverse DFT per residue.

#include "common.hpp"

namespace fno {

static constexpr int kAxThreads = 256;

static inline int axis_cols(int P) { return kAxThreads / P; }

size_t axis_fwd_lds_bytes(int N, int m, int MP) {
  (void)m;
  const int P = N / MP;
  return (size_t)MP * P * axis_cols(P) * sizeof(float2);
}

template <int MP>
__global__ __launch_bounds__(kAxThreads) void fno_fwd_axis(AxisArgs a) {
  extern __shared__ float2 smem[];
  constexpr int LG = ilog2(MP);
  const int tid = threadIdx.x;
  const int N = a.N, m = a.m, P = a.P, C = a.C;
  const int CT = kAxThreads / P;
  const int vol = blockIdx.y;
  const int c0 = blockIdx.x * CT;
  const float2 *ip = a.in + (size_t)vol * N * C;
  float2 *D = smem;  // [MP][P][CT]

  {
    const int r = tid / CT, cl = tid - r * CT;
    const int c = c0 + cl;
    if (r < P && c < C) {
      float2 z[MP];
      static_for<0, MP>([&](auto q) { z[q] = ip[(size_t)(r + decltype(q)::value * P) * C + c]; });
      fft_reg<MP, false>(z);
      static_for<0, MP>([&](auto jj) {
        constexpr int j = decltype(jj)::value;
        D[((size_t)j * P + r) * CT + cl] = z[bitrev(j, LG)];
      });
    }
  }
  __syncthreads();
  float2 *op = a.out + (size_t)vol * 2 * m * C;
  for (int v = tid; v < 2 * m * CT; v += kAxThreads) {
    const int ai = v / CT, cl = v - ai * CT;
    const int c = c0 + cl;
    if (c >= C) continue;
    const int k = ai < m ? ai : N - 2 * m + ai;
    const int j = k & (MP - 1);
    const float2 w = a.tw[k];
    const float2 *dp = D + (size_t)j * P * CT + cl;
    float2 acc = dp[(size_t)(P - 1) * CT];
    for (int r = P - 2; r >= 0; --r) acc = cfma(acc, w, dp[(size_t)r * CT]);
    op[(size_t)ai * C + c] = make_float2(acc.x * a.scale, acc.y * a.scale);
  }
}

template <int MP>
__global__ __launch_bounds__(kAxThreads) void fno_inv_axis(AxisArgs a) {
  constexpr int LG = ilog2(MP);
  const int tid = threadIdx.x;
  const int N = a.N, m = a.m, P = a.P, C = a.C;
  const int CT = kAxThreads / P;
  const int vol = blockIdx.y;
  const int r = tid / CT, cl = tid - r * CT;
  const int c = blockIdx.x * CT + cl;
  if (r >= P || c >= C) return;
  const float2 *ip = a.in + (size_t)vol * 2 * m * C;
  float2 *op = a.out + (size_t)vol * N * C;
  const float2 wc = a.tw[(MP * r) & (N - 1)];  // exp(-2 pi i r / P)
  float2 e[MP];
  static_for<0, MP>([&](auto jj) {
    constexpr int j = decltype(jj)::value;
    // branch-free: out-of-corner rows read row 0 and are selected away
    const bool lo = j < m, hi = j >= MP - m;
    const float2 vl = ip[(size_t)(lo ? j : 0) * C + c];
    const float2 vh = ip[(size_t)(hi ? 2 * m - MP + j : 0) * C + c];
    const float2 th = cmul(vh, wc);
    const float2 s = make_float2((lo ? vl.x : 0.f) + (hi ? th.x : 0.f), (lo ? vl.y : 0.f) + (hi ? th.y : 0.f));
    e[j] = cmulc(s, a.tw[(j * r) & (N - 1)]);
  });
  fft_reg<MP, true>(e);
  static_for<0, MP>([&](auto qq) {
    constexpr int q = decltype(qq)::value;
    op[(size_t)(r + q * P) * C + c] = e[bitrev(q, LG)];
  });
}

static const void *axis_kernel(bool fwd, int MP) {
  switch (MP) {
    case 2: return fwd ? (const void *)fno_fwd_axis<2> : (const void *)fno_inv_axis<2>;
    case 4: return fwd ? (const void *)fno_fwd_axis<4> : (const void *)fno_inv_axis<4>;
    case 8: return fwd ? (const void *)fno_fwd_axis<8> : (const void *)fno_inv_axis<8>;
    case 16: return fwd ? (const void *)fno_fwd_axis<16> : (const void *)fno_inv_axis<16>;
    case 32: return fwd ? (const void *)fno_fwd_axis<32> : (const void *)fno_inv_axis<32>;
  }
  return nullptr;
}

hipError_t axis_fwd_prepare(int MP, size_t lds) {
  const void *k = axis_kernel(true, MP);
  if (!k) return hipErrorInvalidValue;
  return raise_lds_cap(k, lds);
}

hipError_t launch_axis_fwd(const AxisArgs &a, int MP, size_t lds, hipStream_t s) {
  FNO_BOUNDS(check_axis(a, true);)
  const void *k = axis_kernel(true, MP);
  if (!k) return hipErrorInvalidValue;
  const int CT = axis_cols(a.P);
  dim3 grid((a.C + CT - 1) / CT, a.nvol);
  void *args[] = {(void *)&a};
  return hipLaunchKernel(k, grid, dim3(kAxThreads), args, lds, s);
}

hipError_t launch_axis_inv(const AxisArgs &a, int MP, hipStream_t s) {
  FNO_BOUNDS(check_axis(a, false);)
  const void *k = axis_kernel(false, MP);
  if (!k) return hipErrorInvalidValue;
  const int CT = axis_cols(a.P);
  dim3 grid((a.C + CT - 1) / CT, a.nvol);
  void *args[] = {(void *)&a};
  return hipLaunchKernel(k, grid, dim3(kAxThreads), args, 0, s);
}

}  // namespace fno
