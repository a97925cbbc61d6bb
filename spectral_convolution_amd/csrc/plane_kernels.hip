// plane_kernels.hip - pruned forward / inverse 2D transforms of real planes.
//
// One workgroup (256 threads) per plane. The transforms keep only the
// retained low-frequency modes of the FNO layer (TurboFNO write-up, section
// 2.2 and 2.3: corners in kx, half spectrum in ky) and never form the full
// spectrum.
//
// Pruning by decimation: with MP = next_pow2(m) and P = N / MP, sample n of
// a length-N axis is split as n = r + P q (r < P, q < MP). Forward, for
// every residue r an MP-point DFT over q gives D_r[j]; a retained output k
// is then sum_r w^r D_r[k mod MP] with w = exp(-2 pi i k / N), summed by
// Horner's rule. Inverse (input pruned), the retained inputs are
// pre-multiplied per residue and one MP-point inverse DFT per residue gives
// the P-strided outputs n = r + P q directly.
//
// The MP-point DFTs run in registers (fft_reg.hpp). Along the contiguous
// (real) axis two residues are packed as the real and imaginary parts of one
// complex sequence, so one complex FFT serves two real ones. Rows are read
// straight from global memory in adjacent pairs; the partial spectra of a
// chunk of rows meet in LDS for the Horner combine; the row spectra of the
// whole plane (H x m2 complex) stay in LDS for the column stage.

#include "common.hpp"

namespace fno {

static constexpr int kThreads = 256;

static size_t fwd_lds_for(int H, int W, int m2, int MP, int CH) {
  const int PW = W / MP;
  const size_t rowd = (size_t)(MP / 2 + 1) * CH * (PW + 1);
  const size_t cold = (size_t)H * m2;
  const size_t dreg = rowd > cold ? rowd : cold;
  return (dreg + (size_t)H * (m2 + 1)) * sizeof(float2);
}

// Rows per chunk of the row stage: enough units for all threads, halved
// while the LDS footprint exceeds the 160 KiB a workgroup may hold.
int plane_fwd_chunk_rows(int H, int W, int m1, int m2, int MP) {
  (void)m1;
  const int Q = (W / MP) >> 1;
  int ch = kThreads / Q;
  if (ch > H) ch = H;
  while (ch > 1 && fwd_lds_for(H, W, m2, MP, ch) > 160 * 1024) ch >>= 1;
  return ch;
}

size_t plane_fwd_lds_bytes(int H, int W, int m1, int m2, int MP) {
  return fwd_lds_for(H, W, m2, MP, plane_fwd_chunk_rows(H, W, m1, m2, MP));
}

size_t plane_inv_lds_bytes(int H, int W, int m1, int m2, int MP) {
  (void)MP;
  return ((size_t)2 * m1 * m2 + (size_t)H * (m2 + 1) + W + H) * sizeof(float2);
}

template <int MP, int DT>
__global__ __launch_bounds__(kThreads) void fno_fwd_plane(PlaneFwdArgs a) {
  extern __shared__ float2 smem[];
  constexpr int LG = ilog2(MP);
  constexpr int KH = MP / 2 + 1;
  const int tid = threadIdx.x;
  const int H = a.H, W = a.W, m1 = a.m1, m2 = a.m2, PH = a.PH, PW = a.PW;
  const int Q = PW >> 1;
  const int CH = a.CH;
  const int PWp = PW + 1, m2p = m2 + 1;
  const size_t rowd = (size_t)KH * CH * PWp, cold = (size_t)H * m2;
  float2 *D = smem;
  float2 *R = smem + (rowd > cold ? rowd : cold);

  const int plane = blockIdx.x;
  const size_t xoff = (size_t)plane * H * W;

  // ---- row stage: r2c along W, outputs ky < m2, into R[h][ky]
  for (int row0 = 0; row0 < H; row0 += CH) {
    if (tid < CH * Q) {
      const int rl = tid / Q, p = tid - rl * Q;
      const size_t rbase = xoff + (size_t)(row0 + rl) * W + 2 * p;
      float2 z[MP];
      static_for<0, MP>([&](auto q) { z[q] = load_pair<DT>(a.x, rbase + (size_t)decltype(q)::value * PW); });
      fft_reg<MP, false>(z);
      // split the packed pair: D_{2p}[k] = Z[k] + conj Z[-k], D_{2p+1}[k] =
      // -i (Z[k] - conj Z[-k]) (both doubled; the 1/2 is folded into scale)
      float2 *d = D + (size_t)rl * PWp + 2 * p;
      static_for<0, KH>([&](auto kk) {
        constexpr int k = decltype(kk)::value;
        const float2 zk = z[bitrev(k, LG)];
        const float2 zm = z[bitrev((MP - k) & (MP - 1), LG)];
        float2 *dk = d + (size_t)k * CH * PWp;
        dk[0] = make_float2(zk.x + zm.x, zk.y - zm.y);
        dk[1] = make_float2(zk.y + zm.y, zm.x - zk.x);
      });
    }
    __syncthreads();
    for (int v = tid; v < CH * m2; v += kThreads) {
      const int k = v / CH, rl = v - k * CH;
      const bool cj = k > MP / 2;
      const int kk = cj ? MP - k : k;
      const float2 w = a.tw_w[k];
      const float2 *dp = D + ((size_t)kk * CH + rl) * PWp;
      float2 acc = dp[PW - 1];
      if (cj) acc.y = -acc.y;
      for (int r = PW - 2; r >= 0; --r) {
        float2 dv = dp[r];
        if (cj) dv.y = -dv.y;
        acc = cfma(acc, w, dv);
      }
      R[(size_t)(row0 + rl) * m2p + k] = acc;
    }
    __syncthreads();
  }

  // ---- column stage: c2c along H on the m2 retained columns, kx corners
  for (int u = tid; u < m2 * PH; u += kThreads) {
    const int r = u / m2, ky = u - r * m2;
    float2 z[MP];
    static_for<0, MP>([&](auto q) { z[q] = R[(size_t)(r + decltype(q)::value * PH) * m2p + ky]; });
    fft_reg<MP, false>(z);
    static_for<0, MP>([&](auto jj) {
      constexpr int j = decltype(jj)::value;
      D[((size_t)j * PH + r) * m2 + ky] = z[bitrev(j, LG)];
    });
  }
  __syncthreads();
  const float sc = a.scale * 0.5f;
  float2 *op = a.out + (size_t)plane * 2 * m1 * m2;
  for (int v = tid; v < 2 * m1 * m2; v += kThreads) {
    const int ai = v / m2, ky = v - ai * m2;
    const int kx = ai < m1 ? ai : H - 2 * m1 + ai;
    const int j = kx & (MP - 1);
    const float2 w = a.tw_h[kx];
    const float2 *dp = D + (size_t)j * PH * m2 + ky;
    float2 acc = dp[(size_t)(PH - 1) * m2];
    for (int r = PH - 2; r >= 0; --r) acc = cfma(acc, w, dp[(size_t)r * m2]);
    op[v] = make_float2(acc.x * sc, acc.y * sc);
  }
}

template <int MP, int DT>
__global__ __launch_bounds__(kThreads) void fno_inv_plane(PlaneInvArgs a) {
  extern __shared__ float2 smem[];
  constexpr int LG = ilog2(MP);
  const int tid = threadIdx.x;
  const int H = a.H, W = a.W, m1 = a.m1, m2 = a.m2, PH = a.PH, PW = a.PW;
  const int m2p = m2 + 1;
  const int K = 2 * m1 * m2;
  float2 *Yh = smem;                       // [2*m1][m2]
  float2 *Zb = Yh + K;                     // [H][m2 + 1]
  float2 *tww = Zb + (size_t)H * m2p;      // [W]
  float2 *twh = tww + W;                   // [H]

  const int plane = blockIdx.x;
  const float2 *ip = a.in + (size_t)plane * K;
  for (int v = tid; v < K; v += kThreads) Yh[v] = ip[v];
  for (int v = tid; v < W; v += kThreads) tww[v] = a.tw_w[v];
  for (int v = tid; v < H; v += kThreads) twh[v] = a.tw_h[v];
  __syncthreads();

  // ---- column stage (input pruned): Z[r + PH q][ky] from the 2*m1 rows
  for (int u = tid; u < m2 * PH; u += kThreads) {
    const int r = u / m2, ky = u - r * m2;
    const float2 wc = twh[(MP * r) & (H - 1)];  // exp(-2 pi i r / PH)
    float2 e[MP];
    static_for<0, MP>([&](auto jj) {
      constexpr int j = decltype(jj)::value;
      float2 s = make_float2(0.f, 0.f);
      if (j < m1) s = Yh[j * m2 + ky];
      if (j >= MP - m1) s = cfma(Yh[(2 * m1 - MP + j) * m2 + ky], wc, s);
      e[j] = cmulc(s, twh[(j * r) & (H - 1)]);
    });
    fft_reg<MP, true>(e);
    static_for<0, MP>([&](auto qq) {
      constexpr int q = decltype(qq)::value;
      Zb[(size_t)(r + q * PH) * m2p + ky] = e[bitrev(q, LG)];
    });
  }
  __syncthreads();

  // ---- row stage (c2r): two residues per unit, one complex inverse FFT
  const int Q = PW >> 1;
  const size_t yoff = (size_t)plane * H * W;
  for (int u = tid; u < H * Q; u += kThreads) {
    const int row = u / Q, p = u - row * Q;
    const int r0 = 2 * p, r1 = r0 + 1;
    const float2 *zr = Zb + (size_t)row * m2p;
    // F_t[j] = g_j Z[j] exp(+2 pi i j r_t / W), g_0 = 1/2, g_j = 1, zero for j >= m2
    float2 f0[MP], f1[MP];
    static_for<0, MP>([&](auto jj) {
      constexpr int j = decltype(jj)::value;
      if (j < m2) {
        float2 zv = zr[j];
        if (j == 0) zv = make_float2(0.5f * zv.x, 0.5f * zv.y);
        f0[j] = cmulc(zv, tww[(j * r0) & (W - 1)]);
        f1[j] = cmulc(zv, tww[(j * r1) & (W - 1)]);
      } else {
        f0[j] = make_float2(0.f, 0.f);
        f1[j] = make_float2(0.f, 0.f);
      }
    });
    // G[j] = (F0[j] + conj F0[-j]) + i (F1[j] + conj F1[-j]); IDFT(G) = y_r0 + i y_r1
    float2 g[MP];
    static_for<0, MP>([&](auto jj) {
      constexpr int j = decltype(jj)::value;
      constexpr int mj = (MP - j) & (MP - 1);
      const float2 u0 = make_float2(f0[j].x + f0[mj].x, f0[j].y - f0[mj].y);
      const float2 u1 = make_float2(f1[j].x + f1[mj].x, f1[j].y - f1[mj].y);
      g[j] = make_float2(u0.x - u1.y, u0.y + u1.x);
    });
    fft_reg<MP, true>(g);
    const size_t rbase = yoff + (size_t)row * W + r0;
    static_for<0, MP>([&](auto qq) {
      constexpr int q = decltype(qq)::value;
      const float2 v = g[bitrev(q, LG)];
      store_pair<DT>(a.y, rbase + (size_t)q * PW, v.x, v.y);
    });
  }
}

// --------------------------------------------------------------- launchers

template <int DT>
static const void *fwd_kernel_ptr(int MP) {
  switch (MP) {
    case 2: return (const void *)fno_fwd_plane<2, DT>;
    case 4: return (const void *)fno_fwd_plane<4, DT>;
    case 8: return (const void *)fno_fwd_plane<8, DT>;
    case 16: return (const void *)fno_fwd_plane<16, DT>;
    case 32: return (const void *)fno_fwd_plane<32, DT>;
  }
  return nullptr;
}

template <int DT>
static const void *inv_kernel_ptr(int MP) {
  switch (MP) {
    case 2: return (const void *)fno_inv_plane<2, DT>;
    case 4: return (const void *)fno_inv_plane<4, DT>;
    case 8: return (const void *)fno_inv_plane<8, DT>;
    case 16: return (const void *)fno_inv_plane<16, DT>;
    case 32: return (const void *)fno_inv_plane<32, DT>;
  }
  return nullptr;
}

static const void *plane_kernel(bool fwd, int MP, int dtype) {
  switch (dtype) {
    case DT_F32: return fwd ? fwd_kernel_ptr<DT_F32>(MP) : inv_kernel_ptr<DT_F32>(MP);
    case DT_F16: return fwd ? fwd_kernel_ptr<DT_F16>(MP) : inv_kernel_ptr<DT_F16>(MP);
    case DT_BF16: return fwd ? fwd_kernel_ptr<DT_BF16>(MP) : inv_kernel_ptr<DT_BF16>(MP);
  }
  return nullptr;
}

hipError_t plane_fwd_prepare(int MP, int dtype, size_t lds) {
  const void *k = plane_kernel(true, MP, dtype);
  if (!k) return hipErrorInvalidValue;
  return hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

hipError_t plane_inv_prepare(int MP, int dtype, size_t lds) {
  const void *k = plane_kernel(false, MP, dtype);
  if (!k) return hipErrorInvalidValue;
  return hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

hipError_t launch_plane_fwd(const PlaneFwdArgs &a, int MP, int dtype, size_t lds, hipStream_t s) {
  const void *k = plane_kernel(true, MP, dtype);
  if (!k) return hipErrorInvalidValue;
  void *args[] = {(void *)&a};
  return hipLaunchKernel(k, dim3(a.nplanes), dim3(kThreads), args, lds, s);
}

hipError_t launch_plane_inv(const PlaneInvArgs &a, int MP, int dtype, size_t lds, hipStream_t s) {
  const void *k = plane_kernel(false, MP, dtype);
  if (!k) return hipErrorInvalidValue;
  void *args[] = {(void *)&a};
  return hipLaunchKernel(k, dim3(a.nplanes), dim3(kThreads), args, lds, s);
}

}  // namespace fno
