// plane_valu.hpp - device bodies of the VALU plane transforms (pruned
// register FFTs), one 256-thread workgroup's share of planes per call, so
// that both the stand-alone kernels and the single-launch layer run them.
#pragma once

#include "plane_common.hpp"

namespace fno {

// Row-stage chunk: CH = 256 / T rows (T = PW / RPT threads per row) staged in
// LDS as fp32 with a row pitch of W + 2T floats, which spreads the 16 rows x
// T lanes of one 8-byte LDS access over all 32 banks.
__host__ __device__ inline int chunk_rows(int W, int MP) { return kThreads / ((W / MP) / 2); }
__host__ __device__ inline int stage_pitch(int W, int MP) {
  const int T = (W / MP) / 2;
  return W + (T < 16 ? 2 * T : 0);
}

// elements per 16-byte (or smaller) vector of the coalesced chunk copies
template <int MP, int DT>
struct ChunkVec {
  static constexpr int kMax = DT == DT_F32 ? 4 : 8;
  static constexpr int V = kMax < 2 * MP ? kMax : 2 * MP;  // divides the 2*MP elements per thread
  static constexpr int N = 2 * MP / V;                      // vectors per thread per chunk
};

// V consecutive storage elements (V * element size = 4, 8 or 16 bytes) as
// one load, widened to fp32
template <int DT, int V>
__device__ __forceinline__ void gload_vec(const void *base, size_t idx, float (&v)[V]) {
  if constexpr (DT == DT_F32) {
    static_assert(V == 2 || V == 4, "fp32 vector of 2 or 4");
    if constexpr (V == 4) {
      const float4 u = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(base) + idx);
      v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
    } else {
      const float2 u = *reinterpret_cast<const float2 *>(reinterpret_cast<const float *>(base) + idx);
      v[0] = u.x; v[1] = u.y;
    }
  } else {
    static_assert(V == 2 || V == 4 || V == 8, "16-bit vector of 2, 4 or 8");
    const uint16_t *p = reinterpret_cast<const uint16_t *>(base) + idx;
    uint32_t w[V / 2];
    if constexpr (V == 8) {
      const uint4 u = *reinterpret_cast<const uint4 *>(p);
      w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
    } else if constexpr (V == 4) {
      const uint2 u = *reinterpret_cast<const uint2 *>(p);
      w[0] = u.x; w[1] = u.y;
    } else {
      w[0] = *reinterpret_cast<const uint32_t *>(p);
    }
    static_for<0, V / 2>([&](auto cc) {
      constexpr int c = decltype(cc)::value;
      if constexpr (DT == DT_F16) {
        const half2_t h = __builtin_bit_cast(half2_t, w[c]);
        v[2 * c] = (float)h.x;
        v[2 * c + 1] = (float)h.y;
      } else {
        v[2 * c] = __uint_as_float(w[c] << 16);
        v[2 * c + 1] = __uint_as_float(w[c] & 0xffff0000u);
      }
    });
  }
}

template <int DT, int V>
__device__ __forceinline__ void gstore_vec(void *base, size_t idx, const float (&v)[V]) {
  if constexpr (DT == DT_F32 && V == 4) {
    *reinterpret_cast<float4 *>(reinterpret_cast<float *>(base) + idx) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    static_for<0, V / 2>([&](auto cc) {
      constexpr int c = decltype(cc)::value;
      store_pair<DT>(base, idx + 2 * c, v[2 * c], v[2 * c + 1]);
    });
  }
}

// Planes blk * ppw .. + ppw - 1 (one 256-thread workgroup); LDS at smem.
template <int MP, int DT>
__device__ __forceinline__ void fwd_plane_block(const PlaneFwdArgs &a, int blk, float2 *smem) {
  constexpr int LG = ilog2(MP);
  const int tid = threadIdx.x;
  const int H = a.H, W = a.W, m1 = a.m1, m2 = a.m2, PH = a.PH, PW = a.PW, ppw = a.ppw;
  const int m2p = m2 + 1;
  float2 *tww = smem;
  float2 *twh = tww + W;
  float2 *R = twh + H;                                        // [ppw][H][m2 + 1]
  float *stage = reinterpret_cast<float *>(R + (size_t)ppw * H * m2p);  // [CH][pitch]
  for (int v = tid; v < W; v += kThreads) tww[v] = a.tw_w[v];
  for (int v = tid; v < H; v += kThreads) twh[v] = a.tw_h[v];
  const int plane0 = blk * ppw;
  const int nlive = min(ppw, a.nplanes - plane0);

  // ---- row stage: r2c along W, outputs ky < m2, into R. Rows are copied
  // chunk by chunk into LDS with coalesced 16-byte accesses (the next chunk's
  // loads are in flight while the current one is transformed); a thread then
  // takes two adjacent residues of one row. Each output is reduced over the
  // T threads of its row and stored as soon as it is formed.
  using CV = ChunkVec<MP, DT>;
  const int T = PW / 2;
  const int CH = kThreads / T, pitch = stage_pitch(W, MP);
  const int nrows = nlive * H;
  const int nchunks = (nrows + CH - 1) / CH;
  const size_t gbase = (size_t)plane0 * H * W;
  float pre[CV::N][CV::V];
  auto fetch = [&](int c) {
    static_for<0, CV::N>([&](auto vv) {
      constexpr int v = decltype(vv)::value;
      const int e = (v * kThreads + tid) * CV::V;  // element within the chunk
      const int row = c * CH + e / W;
      // rows past the workgroup's planes read row 0 instead (branch-free;
      // their values are never used)
      const size_t off = row < nrows ? (size_t)c * CH * W + e : (size_t)(e % W);
      gload_vec<DT, CV::V>(a.x, gbase + off, pre[v]);
    });
  };
  fetch(0);
  for (int c = 0; c < nchunks; ++c) {
    static_for<0, CV::N>([&](auto vv) {
      constexpr int v = decltype(vv)::value;
      const int e = (v * kThreads + tid) * CV::V;
      const int rl = e / W, col = e - rl * W;
      float2 *dst = reinterpret_cast<float2 *>(stage + rl * pitch + col);
      static_for<0, CV::V / 2>([&](auto ii) {
        constexpr int i = decltype(ii)::value;
        dst[i] = make_float2(pre[v][2 * i], pre[v][2 * i + 1]);
      });
    });
    __syncthreads();
    if (c + 1 < nchunks) fetch(c + 1);
    const int rl = tid / T, t = tid - rl * T;
    const int grow = c * CH + rl;
    const bool live = grow < nrows;
    const int pl = grow / H, row = grow - pl * H;
    const int r0 = 2 * t;
    float2 za[MP];
    const float *src = stage + rl * pitch + r0;
    static_for<0, MP>([&](auto qq) {
      constexpr int q = decltype(qq)::value;
      za[q] = *reinterpret_cast<const float2 *>(src + q * PW);
    });
    fft_reg<MP, false>(za);
    float2 S[MP];
    static_for<0, MP>([&](auto kk) {
      constexpr int k = decltype(kk)::value;
      constexpr int ik = bitrev(k, LG), im = bitrev((MP - k) & (MP - 1), LG);
      // two real spectra from one complex one (both doubled; 1/2 folded into scale)
      const float2 A = za[ik], Am = za[im];
      const float2 d0 = make_float2(A.x + Am.x, A.y - Am.y);
      const float2 d1 = make_float2(A.y + Am.y, Am.x - A.x);
      const float2 acc = cfma(d1, tww[k], d0);
      S[k] = k < m2 ? cmul(acc, tww[(r0 * k) & (W - 1)]) : make_float2(0.f, 0.f);
    });
    group_sum_all(S, T);
    if (live && t == 0) {
      float2 *rr = R + ((size_t)pl * H + row) * m2p;
      static_for<0, MP>([&](auto kk) {
        constexpr int k = decltype(kk)::value;
        if (k < m2) rr[k] = S[k];
      });
    }
    __syncthreads();
  }

  // ---- column stage: c2c along H on the m2 retained columns, kx corners
  fwd_col_stage<MP>(R, nlive, plane0, H, m1, m2, PH, a.rc, twh, a.out, a.scale * 0.5f);
}

template <int MP, int DT>
__device__ __forceinline__ void inv_plane_block(const PlaneInvArgs &a, int blk, float2 *smem) {
  constexpr int LG = ilog2(MP);
  const int tid = threadIdx.x;
  const int H = a.H, W = a.W, m1 = a.m1, m2 = a.m2, PH = a.PH, PW = a.PW, ppw = a.ppw;
  const int m2p = m2 + 1;
  const int K = 2 * m1 * m2;
  float2 *tww = smem;                      // [W]
  float2 *twh = tww + W;                   // [H]
  float2 *Yh = twh + H;                    // [ppw][K]
  float2 *Zb = Yh + (size_t)ppw * K;       // [ppw][H][m2 + 1]
  float *stage = reinterpret_cast<float *>(Zb + (size_t)ppw * H * m2p);  // [CH][pitch]
  const int plane0 = blk * ppw;
  const int nlive = min(ppw, a.nplanes - plane0);
  for (int v = tid; v < W; v += kThreads) tww[v] = a.tw_w[v];
  for (int v = tid; v < H; v += kThreads) twh[v] = a.tw_h[v];
  for (int v = tid; v < nlive * K; v += kThreads) Yh[v] = a.in[(size_t)plane0 * K + v];
  __syncthreads();

  // ---- column stage (input pruned): Z[r + PH q][ky] from the 2*m1 rows
  inv_col_stage<MP>(Yh, Zb, nlive, H, m1, m2, PH, twh);
  __syncthreads();

  // ---- row stage (c2r): two adjacent residues per thread in one complex
  // inverse FFT (Hermitian parts as real and imaginary parts). Results go to
  // an LDS chunk of rows, which is then written out with coalesced stores.
  using CV = ChunkVec<MP, DT>;
  const int T = PW / 2;
  const int CH = kThreads / T, pitch = stage_pitch(W, MP);
  const int nrows = nlive * H;
  const int nchunks = (nrows + CH - 1) / CH;
  const size_t gbase = (size_t)plane0 * H * W;
  for (int c = 0; c < nchunks; ++c) {
    const int rl = tid / T, t = tid - rl * T;
    const int grow = c * CH + rl;
    if (grow < nrows) {
      const int pl = grow / H, row = grow - pl * H;
      const float2 *zr = Zb + ((size_t)pl * H + row) * m2p;
      const int ra = 2 * t, rb = ra + 1;
      // F_t[j] = g_j Z[j] exp(+2 pi i j r_t / W), g_0 = 1/2, g_j = 1; zero for j >= m2
      float2 fa[MP], fb[MP], g[MP];
      static_for<0, MP>([&](auto jj) {
        constexpr int j = decltype(jj)::value;
        if (j < m2) {
          float2 zv = zr[j];
          if (j == 0) zv = make_float2(0.5f * zv.x, 0.5f * zv.y);
          fa[j] = cmulc(zv, tww[(j * ra) & (W - 1)]);
          fb[j] = cmulc(zv, tww[(j * rb) & (W - 1)]);
        } else {
          fa[j] = make_float2(0.f, 0.f);
          fb[j] = make_float2(0.f, 0.f);
        }
      });
      static_for<0, MP>([&](auto jj) {
        constexpr int j = decltype(jj)::value;
        constexpr int mj = (MP - j) & (MP - 1);
        const float2 u0 = make_float2(fa[j].x + fa[mj].x, fa[j].y - fa[mj].y);
        const float2 u1 = make_float2(fb[j].x + fb[mj].x, fb[j].y - fb[mj].y);
        g[j] = make_float2(u0.x - u1.y, u0.y + u1.x);
      });
      fft_reg<MP, true>(g);
      float *dst = stage + rl * pitch + ra;
      static_for<0, MP>([&](auto qq) {
        constexpr int q = decltype(qq)::value;
        *reinterpret_cast<float2 *>(dst + q * PW) = g[bitrev(q, LG)];
      });
    }
    __syncthreads();
    static_for<0, CV::N>([&](auto vv) {
      constexpr int v = decltype(vv)::value;
      const int e = (v * kThreads + tid) * CV::V;
      const int rl2 = e / W, col = e - rl2 * W;
      if (c * CH + rl2 < nrows) {
        float o[CV::V];
        const float2 *sp = reinterpret_cast<const float2 *>(stage + rl2 * pitch + col);
        static_for<0, CV::V / 2>([&](auto ii) {
          constexpr int i = decltype(ii)::value;
          const float2 w2 = sp[i];
          o[2 * i] = w2.x;
          o[2 * i + 1] = w2.y;
        });
        gstore_vec<DT, CV::V>(a.y, gbase + (size_t)c * CH * W + e, o);
      }
    });
    __syncthreads();
  }
}

}  // namespace fno
