// plane_common.hpp - device pieces shared by the plane transforms: lane-group
// sums and the column stages (pruned c2c FFTs along the non-contiguous axis
// of a plane, one thread per (column, residue)).
#pragma once

#include "common.hpp"

namespace fno {

static constexpr int kThreads = 256;

// the value held by another lane of the same 16-lane row (DPP control CTRL)
template <int CTRL>
__device__ __forceinline__ float dpp_get(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over each group of T consecutive lanes (T a power of two <= 64, groups
// aligned to multiples of T); every lane of a group receives the group sum.
// Butterfly order: lane ^ 1, ^ 2 (quad permutes), ^ 4 (half-row mirror, valid
// once quads agree), ^ 8 (row mirror), then ^ 16, ^ 32 through LDS permutes.
__device__ __forceinline__ float lane_group_sum(float v, int T) {
  if (T >= 2) v += dpp_get<0xB1>(v);    // quad_perm [1,0,3,2]
  if (T >= 4) v += dpp_get<0x4E>(v);    // quad_perm [2,3,0,1]
  if (T >= 8) v += dpp_get<0x141>(v);   // row_half_mirror
  if (T >= 16) v += dpp_get<0x140>(v);  // row_mirror
  if (T >= 32) v += __shfl_xor(v, 16, 64);
  if (T >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

__device__ __forceinline__ float2 lane_group_sum(float2 v, int T) {
  return make_float2(lane_group_sum(v.x, T), lane_group_sum(v.y, T));
}

template <int CTRL, int N>
__device__ __forceinline__ void dpp_add_all(float2 (&S)[N]) {
  static_for<0, N>([&](auto kk) {
    constexpr int k = decltype(kk)::value;
    S[k].x += dpp_get<CTRL>(S[k].x);
    S[k].y += dpp_get<CTRL>(S[k].y);
  });
}

template <int N>
__device__ __forceinline__ void shfl_add_all(float2 (&S)[N], int s) {
  static_for<0, N>([&](auto kk) {
    constexpr int k = decltype(kk)::value;
    S[k].x += __shfl_xor(S[k].x, s, 64);
    S[k].y += __shfl_xor(S[k].y, s, 64);
  });
}

// lane_group_sum applied to a whole array: one uniform branch per level
template <int N>
__device__ __forceinline__ void group_sum_all(float2 (&S)[N], int T) {
  if (T >= 2) dpp_add_all<0xB1>(S);
  if (T >= 4) dpp_add_all<0x4E>(S);
  if (T >= 8) dpp_add_all<0x141>(S);
  if (T >= 16) dpp_add_all<0x140>(S);
  if (T >= 32) shfl_add_all(S, 16);
  if (T >= 64) shfl_add_all(S, 32);
}

// Forward column stage. R holds, per plane, the row spectra [H][m2 + 1]
// (complex fp32, LDS). For every retained column ky and every corner row kx
// the output sum_h R[h][ky] exp(-2 pi i kx h / H) is formed by decimation
// (residues r < PH of h = r + PH q, one MP-point FFT per residue and
// thread, residue sum by a butterfly over the PH lanes of the column) and
// written, times sc, to out[plane][kx row][ky] (complex fp32, global).
template <int MP>
__device__ __forceinline__ void fwd_col_stage(const float2 *R, int nlive, int plane0, int H, int m1, int m2,
                                              int PH, int rc, const float2 *twh, float2 *out, float sc) {
  // One residue per thread (PH <= 64 lanes per column); for MP <= 2, where
  // PH can exceed 64, RC residues per thread accumulate before the reduction.
  const int RC = rc, Tc = PH / RC;
  const int K = 2 * m1 * m2;
  const int m2p = m2 + 1;
  const int tid = threadIdx.x;
  constexpr int LG = ilog2(MP);
  for (int u = tid; u < nlive * m2 * Tc; u += kThreads) {
    const int g = u / Tc, t = u - g * Tc;
    const int pl = g / m2, ky = g - pl * m2;
    const bool live = true;
    const float2 *col = R + (size_t)pl * H * m2p + ky;
    float2 *op = out + (size_t)(live ? plane0 + pl : 0) * K + ky;
    // corner 0: kx = j (j < m1) -> row j; corner 1: kx = H - MP + j
    // (j >= MP - m1) -> row 2*m1 - MP + j
    if constexpr (MP > 2) {
      // one residue per thread; the two corners are formed and reduced in turn
      const int r = t;
      float2 z[MP];
      static_for<0, MP>([&](auto qq) {
        constexpr int q = decltype(qq)::value;
        z[q] = col[(size_t)(r + q * PH) * m2p];
      });
      fft_reg<MP, false>(z);
      float2 O[MP];
      static_for<0, MP>([&](auto jj) {
        constexpr int j = decltype(jj)::value;
        O[j] = j < m1 ? cmul(z[bitrev(j, LG)], twh[(j * r) & (H - 1)]) : make_float2(0.f, 0.f);
      });
      group_sum_all(O, Tc);
      if (live && t == 0)
        static_for<0, MP>([&](auto jj) {
          constexpr int j = decltype(jj)::value;
          if (j < m1) op[(size_t)j * m2] = make_float2(O[j].x * sc, O[j].y * sc);
        });
      static_for<0, MP>([&](auto jj) {
        constexpr int j = decltype(jj)::value;
        O[j] = j >= MP - m1 ? cmul(z[bitrev(j, LG)], twh[((H - MP + j) * r) & (H - 1)]) : make_float2(0.f, 0.f);
      });
      group_sum_all(O, Tc);
      if (live && t == 0)
        static_for<0, MP>([&](auto jj) {
          constexpr int j = decltype(jj)::value;
          if (j >= MP - m1) op[(size_t)(2 * m1 - MP + j) * m2] = make_float2(O[j].x * sc, O[j].y * sc);
        });
    } else {
      // MP <= 2: RC residues per thread accumulate first
      float2 Olo[MP], Ohi[MP];
      static_for<0, MP>([&](auto jj) {
        Olo[decltype(jj)::value] = make_float2(0.f, 0.f);
        Ohi[decltype(jj)::value] = make_float2(0.f, 0.f);
      });
      for (int rr = 0; rr < RC; ++rr) {
        const int r = t * RC + rr;
        float2 z[MP];
        static_for<0, MP>([&](auto qq) {
          constexpr int q = decltype(qq)::value;
          z[q] = col[(size_t)(r + q * PH) * m2p];
        });
        fft_reg<MP, false>(z);
        static_for<0, MP>([&](auto jj) {
          constexpr int j = decltype(jj)::value;
          const float2 d = z[bitrev(j, LG)];
          if (j < m1) Olo[j] = cfma(d, twh[(j * r) & (H - 1)], Olo[j]);
          if (j >= MP - m1) Ohi[j] = cfma(d, twh[((H - MP + j) * r) & (H - 1)], Ohi[j]);
        });
      }
      static_for<0, MP>([&](auto jj) {
        constexpr int j = decltype(jj)::value;
        if (j < m1) {
          float2 v = Olo[j];
          v = lane_group_sum(v, Tc);
          if (live && t == 0) op[(size_t)j * m2] = make_float2(v.x * sc, v.y * sc);
        }
        if (j >= MP - m1) {
          float2 v = Ohi[j];
          v = lane_group_sum(v, Tc);
          if (live && t == 0) op[(size_t)(2 * m1 - MP + j) * m2] = make_float2(v.x * sc, v.y * sc);
        }
      });
    }
  }
}

// Inverse column stage (input pruned). Yh holds, per plane, the 2*m1 x m2
// retained modes (LDS); writes Z[h][ky] = sum over the corner rows of
// Yh exp(+2 pi i kx h / H) into Zb [H][m2 + 1] (LDS), one MP-point inverse
// FFT per (column, residue).
template <int MP>
__device__ __forceinline__ void inv_col_stage(const float2 *Yh, float2 *Zb, int nlive, int H, int m1, int m2, int PH,
                                              const float2 *twh) {
  const int m2p = m2 + 1;
  const int K = 2 * m1 * m2;
  const int tid = threadIdx.x;
  constexpr int LG = ilog2(MP);
  for (int u = tid; u < nlive * PH * m2; u += kThreads) {
    const int g = u / m2, ky = u - g * m2;
    const int pl = g / PH, r = g - pl * PH;
    const float2 *yp = Yh + (size_t)pl * K + ky;
    const float2 wc = twh[(MP * r) & (H - 1)];  // exp(-2 pi i r / PH)
    float2 e[MP];
    static_for<0, MP>([&](auto jj) {
      constexpr int j = decltype(jj)::value;
      float2 s = make_float2(0.f, 0.f);
      if (j < m1) s = yp[j * m2];
      if (j >= MP - m1) s = cfma(yp[(2 * m1 - MP + j) * m2], wc, s);
      e[j] = cmulc(s, twh[(j * r) & (H - 1)]);
    });
    fft_reg<MP, true>(e);
    float2 *zp = Zb + (size_t)pl * H * m2p + ky;
    static_for<0, MP>([&](auto qq) {
      constexpr int q = decltype(qq)::value;
      zp[(size_t)(r + q * PH) * m2p] = e[bitrev(q, LG)];
    });
  }
}

}  // namespace fno
