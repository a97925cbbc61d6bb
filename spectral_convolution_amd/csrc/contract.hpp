// contract.hpp - the per-mode complex channel contraction on MFMA (device
// body, shared by the stand-alone kernel and the single-launch layer).
//
// For every retained mode k: Yh[k] (B x Co) = Xh[k] (B x Ci) * W[k] (Ci x Co),
// complex, no conjugation, fp32 accumulation (TurboFNO write-up, section
// 2.2: the einsum "xyij,xyik->xyjk" with a (modes_x, modes_y, in, out)
// weight; section 3.2 runs it on matrix cores). The complex product is
// lowered to real MFMA products: Yr = Xr Wr + (-Xi) Wi, Yi = Xr Wi + Xi Wr.
//
// Instruction: v_mfma_f32_4x4x1_16b_f32 (16 independent 4x4 outer-product
// blocks per wave). The 16 blocks are 16 consecutive modes, so every lane
// group reads consecutive modes and all global traffic is coalesced in the
// library's natural layouts: Xh and Yh plane-major [b][c][k], W mode-major
// [k][i][o]. Lane l works on mode k0 + l/4; as the A operand it carries
// batch row b0 + 4*bb + l%4, as the B operand four consecutive output
// channels o0 + 4*(l%4) + ob (ob = 0..3, one MFMA each). A wave covers
// 16 modes x (4*BB) batch rows x 16 output channels; W is read once per
// batch tile.

#pragma once

#include "common.hpp"

namespace fno {

template <int BB>
struct Frag {
  float ar[BB], ai[BB], an[BB];
  float wr[4], wi[4];
};

// four consecutive complex weights (vector load; idx a multiple of 4)
template <int DT>
__device__ __forceinline__ void load_w4v(const void *w, size_t idx, float (&re)[4], float (&im)[4]) {
  if constexpr (DT == DT_F32) {
    const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(w) + 2 * idx);
    const float4 u = p[0], v = p[1];
    re[0] = u.x; im[0] = u.y; re[1] = u.z; im[1] = u.w;
    re[2] = v.x; im[2] = v.y; re[3] = v.z; im[3] = v.w;
  } else {
    const uint4 u = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(w) + 2 * idx);
    const uint32_t q[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if constexpr (DT == DT_F16) {
        half2_t h = __builtin_bit_cast(half2_t, q[t]);
        re[t] = (float)h.x;
        im[t] = (float)h.y;
      } else {
        re[t] = __uint_as_float(q[t] << 16);
        im[t] = __uint_as_float(q[t] & 0xffff0000u);
      }
    }
  }
}

// Operands of one input channel i. Lanes whose batch row, mode or output
// channel is out of range read element 0 instead: their values only enter
// products of outputs that are never stored (the 4x4 blocks are per mode,
// rows per batch row, columns per output channel), so they need no zeroing,
// and no load waits for an earlier one's value.
template <int BB, int DT, bool VEC>
__device__ __forceinline__ void load_frag(const ContractArgs &a, int i, int mode, bool mode_ok, int b0, int nn,
                                          int ol, int nw, Frag<BB> &f) {
  const int K = a.K, Ci = a.Ci, Co = a.Co, B = a.B;
#pragma unroll
  for (int bb = 0; bb < BB; ++bb) {
    const int b = b0 + 4 * bb + nn;
    const bool ok = mode_ok && b < B;
    const float2 xv = a.xh[ok ? ((size_t)b * Ci + i) * K + mode : 0];
    f.ar[bb] = xv.x;
    f.ai[bb] = xv.y;
  }
  const size_t widx = ((size_t)(mode_ok ? mode : 0) * Ci + i) * Co + ol;
  if constexpr (VEC) {
    load_w4v<DT>(a.w, nw == 4 ? widx : 0, f.wr, f.wi);
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float2 v = load_pair<DT>(a.w, 2 * (t < nw ? widx + t : 0));
      f.wr[t] = v.x;
      f.wi[t] = v.y;
    }
  }
}

// The input-channel sum is split over the S waves of a workgroup (wave s
// takes channels [s*Ci/S, (s+1)*Ci/S)); each wave keeps the operands of its
// next channels in flight while the MFMAs of the current one run. Partial
// sums meet in LDS, and each wave adds up and stores a share of them.
// VEC: Co is a multiple of 4, each lane's four weights load as one vector.
// Tile (bx, by, bz) = (16-mode block, batch tile of 4 BB rows, 16-channel
// output tile) on the first S waves of the calling workgroup (wave index
// below S); red: LDS for the partial sums when S > 1.
template <int BB, int DT, bool VEC>
__device__ __forceinline__ void contract_tile(const ContractArgs &a, int bx, int by, int bz, int S, float *red) {
  const int lane = threadIdx.x & 63, s = threadIdx.x >> 6;
  const int blk = lane >> 2, nn = lane & 3;
  const int K = a.K, Ci = a.Ci, Co = a.Co, B = a.B;
  const int mode = bx * 16 + blk;
  const int b0 = by * 4 * BB;
  const int o0 = bz * 16;
  const bool mode_ok = mode < K;
  const int ol = o0 + 4 * nn;  // first of this lane's 4 output channels
  const int nw = mode_ok ? min(4, max(0, Co - ol)) : 0;
  const int i0 = (Ci * s) / S, i1 = (Ci * (s + 1)) / S;

  v4f accr[BB][4], acci[BB][4];
#pragma unroll
  for (int bb = 0; bb < BB; ++bb)
#pragma unroll
    for (int ob = 0; ob < 4; ++ob) {
      accr[bb][ob] = v4f{0.f, 0.f, 0.f, 0.f};
      acci[bb][ob] = v4f{0.f, 0.f, 0.f, 0.f};
    }

  // A ring of D + 1 channels' operands in flight: channel i's products run
  // while channels i + 1 .. i + D load, and the slot just used is refilled
  // with channel i + D + 1. Loads are unconditional (clamped to the last
  // channel; repeats are never multiplied) so the compiler's waits count
  // them exactly.
  constexpr int D = BB == 1 ? 3 : BB == 2 ? 2 : 1;
  if (i0 < i1) {
    Frag<BB> ring[D + 1];
#pragma unroll
    for (int k = 0; k <= D; ++k) load_frag<BB, DT, VEC>(a, min(i0 + k, i1 - 1), mode, mode_ok, b0, nn, ol, nw, ring[k]);
    for (int i = i0; i < i1; i += D + 1) {
#pragma unroll
      for (int k = 0; k <= D; ++k) {
        Frag<BB> &cur = ring[k];
        if (i + k < i1) {
#pragma unroll
          for (int bb = 0; bb < BB; ++bb) cur.an[bb] = -cur.ai[bb];
#pragma unroll
          for (int bb = 0; bb < BB; ++bb)
#pragma unroll
            for (int ob = 0; ob < 4; ++ob) {
              accr[bb][ob] = __builtin_amdgcn_mfma_f32_4x4x1f32(cur.ar[bb], cur.wr[ob], accr[bb][ob], 0, 0, 0);
              accr[bb][ob] = __builtin_amdgcn_mfma_f32_4x4x1f32(cur.an[bb], cur.wi[ob], accr[bb][ob], 0, 0, 0);
              acci[bb][ob] = __builtin_amdgcn_mfma_f32_4x4x1f32(cur.ar[bb], cur.wi[ob], acci[bb][ob], 0, 0, 0);
              acci[bb][ob] = __builtin_amdgcn_mfma_f32_4x4x1f32(cur.ai[bb], cur.wr[ob], acci[bb][ob], 0, 0, 0);
            }
        }
        load_frag<BB, DT, VEC>(a, min(i + k + D + 1, i1 - 1), mode, mode_ok, b0, nn, ol, nw, cur);
      }
    }
  }

  // accumulator register j of lane l holds block l/4, row j, column l%4:
  // mode, batch row b0 + 4 bb + j, output channel ol + ob
  if (S == 1) {
    if (!mode_ok) return;
#pragma unroll
    for (int bb = 0; bb < BB; ++bb)
#pragma unroll
      for (int ob = 0; ob < 4; ++ob) {
        const int o = ol + ob;
        if (o >= Co) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int b = b0 + 4 * bb + j;
          if (b < B) a.yh[((size_t)b * Co + o) * K + mode] = make_float2(accr[bb][ob][j], acci[bb][ob][j]);
        }
      }
    return;
  }
  // Every wave's partial sums -> LDS red[wave][pair][re / im][lane], pair =
  // (bb, ob, j); then wave s adds up pairs [s NP / S, (s + 1) NP / S) over
  // the waves in wave order (results do not depend on timing) and stores
  // them.
  constexpr int NP = BB * 16;  // (re, im) pairs per lane
  {
    float *dst = red + (size_t)s * NP * 2 * 64 + lane;
#pragma unroll
    for (int bb = 0; bb < BB; ++bb)
#pragma unroll
      for (int ob = 0; ob < 4; ++ob)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int q = (bb * 4 + ob) * 4 + j;
          dst[(2 * q) * 64] = accr[bb][ob][j];
          dst[(2 * q + 1) * 64] = acci[bb][ob][j];
        }
  }
  __syncthreads();
  if (!mode_ok) return;
  const int per = NP / S;
  for (int q = s * per; q < (s + 1) * per; ++q) {
    float re = 0.f, im = 0.f;
    for (int w = 0; w < S; ++w) {
      re += red[((size_t)w * NP * 2 + 2 * q) * 64 + lane];
      im += red[((size_t)w * NP * 2 + 2 * q + 1) * 64 + lane];
    }
    const int j = q & 3, ob = (q >> 2) & 3, bb = q >> 4;
    const int o = ol + ob, b = b0 + 4 * bb + j;
    if (o < Co && b < B) a.yh[((size_t)b * Co + o) * K + mode] = make_float2(re, im);
  }
}

}  // namespace fno

namespace fno {

// ------------------------------------------------ adjoint straight from W
//
// The adjoint contraction of the backward pass, Gx[k] (B x Ci) = G[k] (B x
// Co) * W[k]^H, with W read in its forward layout [k][i][o] instead of a
// conjugate-transposed copy. The reduction now runs over o, the contiguous
// index of W, while the MFMA B operand wants output channels i across the
// lanes at one o. Each wave therefore stages W through its own LDS region in
// chunks of 16 reduction steps x 4 of its 16 output channels x its 16 modes
// (8 KB): every (mode, channel) row piece is 16 steps = 128 contiguous bytes,
// read by 8 lanes, so the loads move whole cache lines (smaller pieces,
// which revisit each line, measured slower). The pieces are conjugated and
// written transposed as [mode][step][channel]. Lane (mode, n) holds output
// channels n + 4 ob (ob = 0..3); chunk c of a step block carries channels
// 4 c .. 4 c + 3, i.e. every lane's ob = c, read as one 8-byte word per
// step. The four chunks of a step block share the G operand. Waves never
// share a region, so no workgroup barrier is needed until the partial sums
// of a split reduction meet. The reduction of wave s covers pairs of steps
// [P s / S, P (s + 1) / S), P = Co / 2 (Co even), so step blocks start even
// and 16-byte pieces stay aligned; past the end of its range a wave re-reads
// the final pair (in range) and skips those steps.
struct AdjL {
  static constexpr int RC = 16;        // reduction steps per chunk
  static constexpr int P = 5;          // complex per (mode, step) row: 4 channels + 1 pad (odd: the
                                       // transposing 8-byte stores of 16 lanes hit 32 distinct banks)
  static constexpr int Q = 16 * P + 4;  // complex per mode block (= 4 mod 16: the 8-byte reads of four
                                        // neighbouring modes hit distinct banks)
  static constexpr int WAVE = 16 * Q;  // complex per wave region
  static constexpr int NI = 8;         // load instructions per chunk (8 rows of 128 bytes each)
};

template <int BB>
__device__ __forceinline__ void contract_tile_adj(const ContractArgs &a, int bx, int by, int bz, int S,
                                                  float2 *stg) {
  const int lane = threadIdx.x & 63, s = threadIdx.x >> 6;
  const int blk = lane >> 2, nn = lane & 3;
  // in the adjoint's terms: Cr reduction channels (the layer's Co, the last
  // index of W), No output channels (the layer's Ci, the middle index)
  const int K = a.K, Cr = a.Ci, No = a.Co, B = a.B;
  const int mode = bx * 16 + blk;
  const bool mode_ok = mode < K;
  const int b0 = by * 4 * BB, o0 = bz * 16;
  const int Pp = Cr >> 1;
  const int r0s = 2 * ((Pp * s) / S), r1 = 2 * ((Pp * (s + 1)) / S);
  float2 *Wl = stg + (size_t)s * AdjL::WAVE;
  const float2 *w = reinterpret_cast<const float2 *>(a.w);

  // load instruction j: rows 8 j .. 8 j + 7 = (mode q = row / 4, channel
  // 4 c + row % 4), lane: row 8 j + lane / 8, steps r + 2 (lane % 8) and the
  // next one (clamped to the last pair)
  const int lp = lane & 7, lrow = lane >> 3;
  auto fetch = [&](int r, int c, float4 (&v)[AdjL::NI]) {
    const int rr = min(r + 2 * lp, Cr - 2);
    const int o = o0 + 4 * c + (lrow & 3);
#pragma unroll
    for (int j = 0; j < AdjL::NI; ++j) {
      const int m = bx * 16 + 2 * j + (lrow >> 2);
      const bool ok = m < K && o < No;
      v[j] = *reinterpret_cast<const float4 *>(w + (ok ? ((size_t)m * No + o) * Cr + rr : 0));
    }
  };
  auto put = [&](const float4 (&v)[AdjL::NI]) {
#pragma unroll
    for (int j = 0; j < AdjL::NI; ++j) {
      float2 *d = Wl + (2 * j + (lrow >> 2)) * AdjL::Q + (2 * lp) * AdjL::P + (lrow & 3);
      d[0] = make_float2(v[j].x, -v[j].y);
      d[AdjL::P] = make_float2(v[j].z, -v[j].w);
    }
  };
  // the spectra of G for the steps of a block (A operand: batch rows)
  auto gfetch = [&](int r, float2 (&g)[AdjL::RC][BB]) {
#pragma unroll
    for (int t = 0; t < AdjL::RC; ++t) {
      const int rc = min(r + t, Cr - 1);
#pragma unroll
      for (int bb = 0; bb < BB; ++bb) {
        const int b = b0 + 4 * bb + nn;
        const bool ok = mode_ok && b < B;
        g[t][bb] = a.xh[ok ? ((size_t)b * Cr + rc) * K + mode : 0];
      }
    }
  };

  v4f accr[BB][4], acci[BB][4];
#pragma unroll
  for (int bb = 0; bb < BB; ++bb)
#pragma unroll
    for (int ob = 0; ob < 4; ++ob) {
      accr[bb][ob] = v4f{0.f, 0.f, 0.f, 0.f};
      acci[bb][ob] = v4f{0.f, 0.f, 0.f, 0.f};
    }
  // products of the staged chunk c (first step r; steps past r1 skipped)
  auto compute = [&](int r, int c, const float2 (&g)[AdjL::RC][BB]) {
    const int nst = min(AdjL::RC, r1 - r);
#pragma unroll
    for (int t = 0; t < AdjL::RC; ++t) {
      if (t < nst) {
        const float2 u = Wl[blk * AdjL::Q + t * AdjL::P + nn];
#pragma unroll
        for (int bb = 0; bb < BB; ++bb) {
          const float ar = g[t][bb].x, ai = g[t][bb].y, an = -ai;
          v4f &cr = accr[bb][c], &ci = acci[bb][c];
          cr = __builtin_amdgcn_mfma_f32_4x4x1f32(ar, u.x, cr, 0, 0, 0);
          cr = __builtin_amdgcn_mfma_f32_4x4x1f32(an, u.y, cr, 0, 0, 0);
          ci = __builtin_amdgcn_mfma_f32_4x4x1f32(ar, u.y, ci, 0, 0, 0);
          ci = __builtin_amdgcn_mfma_f32_4x4x1f32(ai, u.x, ci, 0, 0, 0);
        }
      }
    }
  };

  if (r0s < r1) {
    // chunks (r, c) in the order (r0s, 0..3), (r0s + 16, 0..3), ...; every
    // W fetch is unconditional (clamped in range) so the compiler's waits
    // count the loads in flight exactly. G of a step block is requested
    // with the block's second chunk, while that chunk's W is in flight.
    float4 wv[AdjL::NI];
    float2 g[AdjL::RC][BB];
    fetch(r0s, 0, wv);
    for (int r0 = r0s; r0 < r1; r0 += AdjL::RC) {
      const int rn = r0 + AdjL::RC < r1 ? r0 + AdjL::RC : r0;
      put(wv);
      fetch(r0, 1, wv);
      gfetch(r0, g);
      compute(r0, 0, g);
      put(wv);
      fetch(r0, 2, wv);
      compute(r0, 1, g);
      put(wv);
      fetch(r0, 3, wv);
      compute(r0, 2, g);
      put(wv);
      fetch(rn, 0, wv);
      compute(r0, 3, g);
    }
  }

  // accumulator register j of lane l: mode, batch row b0 + 4 bb + j, output
  // channel o0 + n + 4 ob
  if (S == 1) {
    if (!mode_ok) return;
#pragma unroll
    for (int bb = 0; bb < BB; ++bb)
#pragma unroll
      for (int ob = 0; ob < 4; ++ob) {
        const int o = o0 + nn + 4 * ob;
        if (o >= No) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int b = b0 + 4 * bb + j;
          if (b < B) a.yh[((size_t)b * No + o) * K + mode] = make_float2(accr[bb][ob][j], acci[bb][ob][j]);
        }
      }
    return;
  }
  // split reduction: every wave's partial sums go to LDS (the staging
  // regions, once every wave is done with its own), then wave s adds up
  // pairs [s NP / S, (s + 1) NP / S) over the waves in wave order
  constexpr int NP = BB * 16;
  float *red = reinterpret_cast<float *>(stg);
  __syncthreads();
  {
    float *dst = red + (size_t)s * NP * 2 * 64 + lane;
#pragma unroll
    for (int bb = 0; bb < BB; ++bb)
#pragma unroll
      for (int ob = 0; ob < 4; ++ob)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int q = (bb * 4 + ob) * 4 + j;
          dst[(2 * q) * 64] = accr[bb][ob][j];
          dst[(2 * q + 1) * 64] = acci[bb][ob][j];
        }
  }
  __syncthreads();
  if (!mode_ok) return;
  const int per = NP / S;
  for (int q = s * per; q < (s + 1) * per; ++q) {
    float re = 0.f, im = 0.f;
    for (int wq = 0; wq < S; ++wq) {
      re += red[((size_t)wq * NP * 2 + 2 * q) * 64 + lane];
      im += red[((size_t)wq * NP * 2 + 2 * q + 1) * 64 + lane];
    }
    const int j = q & 3, ob = (q >> 2) & 3, bb = q >> 4;
    const int o = o0 + nn + 4 * ob, b = b0 + 4 * bb + j;
    if (o < No && b < B) a.yh[((size_t)b * No + o) * K + mode] = make_float2(re, im);
  }
}

}  // namespace fno
