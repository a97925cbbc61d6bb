// backward.hip - the two kernels of the layer's backward pass that the
// forward path does not already provide.
//
// For a loss with gradient g = dL/dy, every step of the layer is linear, so
// its gradients are the adjoints of the steps in reverse order (the TurboFNO
// write-up, section 4.3, hands the layer to PyTorch autograd through a
// backward function; what it returns is fixed by the forward):
//
//   dx          = inverse( forward(g) * W^H )
//   dw[k][i][o] = N gamma_k sum_b conj(Xs[b][i][k]) Gs[b][o][k]
//
// forward / inverse are the library's own plane transforms (forward already
// scaled by 1/N, inverse with the c2r weights gamma and no scale), so dx is
// the layer itself applied to g with every mode's weight replaced by its
// conjugate transpose. Xs = forward(x), Gs = forward(g); N is the grid size
// and gamma_k the c2r weight of the mode's last-axis index (1 for index 0,
// whose imaginary part never reaches y, 2 otherwise).
//
// fno_conj_transpose forms W^H; fno_grad_w is the per-mode batch reduction.

#include "common.hpp"

namespace fno {

// ------------------------------------------------------- W^H = conj(W)^T

// conjugate of one (re, im) element: the sign bit of the imaginary part
__device__ __forceinline__ uint32_t conj_el(uint32_t v) { return v ^ 0x80000000u; }  // two 16-bit parts
__device__ __forceinline__ uint2 conj_el(uint2 v) { return make_uint2(v.x, v.y ^ 0x80000000u); }  // two fp32

// wh[k][o][i] = conj(w[k][i][o]) through a 32 x 32 LDS tile per workgroup:
// reads run along o, writes along i. Workgroup id = (k, i tile, o tile),
// o tiles fastest.
template <typename E>
__global__ __launch_bounds__(256) void fno_conj_transpose(const E *__restrict__ w, E *__restrict__ wh, int Ci,
                                                          int Co, int nti, int nto) {
  __shared__ E tile[32][33];
  const long id = blockIdx.x;
  const int to = (int)(id % nto), ti = (int)((id / nto) % nti);
  const long k = id / ((long)nto * nti);
  const int o0 = to * 32, i0 = ti * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const E *src = w + (size_t)k * Ci * Co;
  E *dst = wh + (size_t)k * Ci * Co;
#pragma unroll
  for (int r = ty; r < 32; r += 8) {
    const int i = i0 + r, o = o0 + tx;
    if (i < Ci && o < Co) tile[r][tx] = conj_el(src[(size_t)i * Co + o]);
  }
  __syncthreads();
#pragma unroll
  for (int r = ty; r < 32; r += 8) {
    const int o = o0 + r, i = i0 + tx;
    if (o < Co && i < Ci) dst[(size_t)o * Ci + i] = tile[tx][r];
  }
}

hipError_t launch_conj_transpose(const void *w, void *wh, int K, int Ci, int Co, int dtype, hipStream_t s) {
  const int nti = (Ci + 31) / 32, nto = (Co + 31) / 32;
  const long n = (long)K * nti * nto;
  if (n < 1 || n > 0x7fffffffL) return hipErrorInvalidValue;
  if (dtype == DT_F32)
    hipLaunchKernelGGL(fno_conj_transpose<uint2>, dim3((unsigned)n), dim3(256), 0, s, (const uint2 *)w, (uint2 *)wh,
                       Ci, Co, nti, nto);
  else
    hipLaunchKernelGGL(fno_conj_transpose<uint32_t>, dim3((unsigned)n), dim3(256), 0, s, (const uint32_t *)w,
                       (uint32_t *)wh, Ci, Co, nti, nto);
  return hipGetLastError();
}

// ------------------------------------------------------------ dw kernel
//
// Instruction: v_mfma_f32_4x4x1_16b_f32, 16 blocks of 4 x 4 per wave, the
// blocks being 16 consecutive modes (so every load of a lane group is a run
// of 16 consecutive complex spectra, coalesced in the plane-major layout).
// The batch is the reduction dimension, one MFMA step per batch row. Lane l
// works on mode k0 + l/4; as the A operand it carries input channel
// i0 + 4 ib + l%4 (conj Xs), as the B operand output channel
// o0 + 4 (l%4) + ob (Gs, ob = 0..3, one MFMA each). In real form
//   Re dw += Xr Gr + Xi Gi,   Im dw += Xr Gi + (-Xi) Gr.
// A wave covers 16 modes x 4 IB input x 16 output channels; the batch sum
// is split over the S waves of a workgroup and met in LDS.

template <int IB>
struct GwFrag {
  float xr[IB], xi[IB], xn[IB];
  float gr[4], gi[4];
};

// Operands of batch row b. Lanes whose mode or channel is out of range read
// element 0: their values reach only outputs that are never stored.
template <int IB>
__device__ __forceinline__ void gw_load(const GradWArgs &a, int b, int mode, bool mode_ok, int i0, int nn, int o0,
                                        GwFrag<IB> &f) {
  const int K = a.K, Ci = a.Ci, Co = a.Co;
#pragma unroll
  for (int ib = 0; ib < IB; ++ib) {
    const int i = i0 + 4 * ib + nn;
    const bool ok = mode_ok && i < Ci;
    const float2 v = a.xs[ok ? ((size_t)b * Ci + i) * K + mode : 0];
    f.xr[ib] = v.x;
    f.xi[ib] = v.y;
  }
#pragma unroll
  for (int ob = 0; ob < 4; ++ob) {
    const int o = o0 + 4 * nn + ob;
    const bool ok = mode_ok && o < Co;
    const float2 v = a.gs[ok ? ((size_t)b * Co + o) * K + mode : 0];
    f.gr[ob] = v.x;
    f.gi[ob] = v.y;
  }
}

template <int IB, int DT>
__global__ __launch_bounds__(512) void fno_grad_w(GradWArgs a) {
  extern __shared__ float red[];
  const int lane = threadIdx.x & 63, s = threadIdx.x >> 6, S = blockDim.x >> 6;
  const int blk = lane >> 2, nn = lane & 3;
  const int K = a.K, Ci = a.Ci, Co = a.Co, B = a.B;
  const int mode = blockIdx.x * 16 + blk;
  const int i0 = blockIdx.y * 4 * IB;
  const int o0 = blockIdx.z * 16;
  const bool mode_ok = mode < K;
  const int b0 = (B * s) / S, b1 = (B * (s + 1)) / S;

  v4f accr[IB][4], acci[IB][4];
#pragma unroll
  for (int ib = 0; ib < IB; ++ib)
#pragma unroll
    for (int ob = 0; ob < 4; ++ob) {
      accr[ib][ob] = v4f{0.f, 0.f, 0.f, 0.f};
      acci[ib][ob] = v4f{0.f, 0.f, 0.f, 0.f};
    }

  // ring of D + 1 batch rows in flight; loads are clamped to the last row of
  // the wave's range (repeats are never multiplied)
  constexpr int D = IB == 1 ? 3 : IB == 2 ? 2 : 1;
  if (b0 < b1) {
    GwFrag<IB> ring[D + 1];
#pragma unroll
    for (int k = 0; k <= D; ++k) gw_load<IB>(a, min(b0 + k, b1 - 1), mode, mode_ok, i0, nn, o0, ring[k]);
    for (int b = b0; b < b1; b += D + 1) {
#pragma unroll
      for (int k = 0; k <= D; ++k) {
        GwFrag<IB> &cur = ring[k];
        if (b + k < b1) {
#pragma unroll
          for (int ib = 0; ib < IB; ++ib) cur.xn[ib] = -cur.xi[ib];
#pragma unroll
          for (int ib = 0; ib < IB; ++ib)
#pragma unroll
            for (int ob = 0; ob < 4; ++ob) {
              accr[ib][ob] = __builtin_amdgcn_mfma_f32_4x4x1f32(cur.xr[ib], cur.gr[ob], accr[ib][ob], 0, 0, 0);
              accr[ib][ob] = __builtin_amdgcn_mfma_f32_4x4x1f32(cur.xi[ib], cur.gi[ob], accr[ib][ob], 0, 0, 0);
              acci[ib][ob] = __builtin_amdgcn_mfma_f32_4x4x1f32(cur.xr[ib], cur.gi[ob], acci[ib][ob], 0, 0, 0);
              acci[ib][ob] = __builtin_amdgcn_mfma_f32_4x4x1f32(cur.xn[ib], cur.gr[ob], acci[ib][ob], 0, 0, 0);
            }
        }
        gw_load<IB>(a, min(b + k + D + 1, b1 - 1), mode, mode_ok, i0, nn, o0, cur);
      }
    }
  }

  // accumulator register j of lane l holds block l/4 (the mode), row j
  // (input channel i0 + 4 ib + j), column l%4 (output channel o0 + 4 (l%4) + ob)
  const float sc = a.scale * ((mode % a.mlast) == 0 ? 1.0f : 2.0f);
  if (S == 1) {
    if (!mode_ok) return;
#pragma unroll
    for (int ib = 0; ib < IB; ++ib)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = i0 + 4 * ib + j;
        if (i >= Ci) continue;
#pragma unroll
        for (int ob = 0; ob < 4; ++ob) {
          const int o = o0 + 4 * nn + ob;
          if (o < Co) store_pair<DT>(a.dw, 2 * (((size_t)mode * Ci + i) * Co + o), sc * accr[ib][ob][j], sc * acci[ib][ob][j]);
        }
      }
    return;
  }
  // partial sums of every wave -> red[wave][pair][re / im][lane], pair =
  // (ib, ob, j); wave s adds up pairs [s NP / S, (s + 1) NP / S) over the
  // waves in wave order (results do not depend on timing) and stores them
  constexpr int NP = IB * 16;
  {
    float *dst = red + (size_t)s * NP * 2 * 64 + lane;
#pragma unroll
    for (int ib = 0; ib < IB; ++ib)
#pragma unroll
      for (int ob = 0; ob < 4; ++ob)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int q = (ib * 4 + ob) * 4 + j;
          dst[(2 * q) * 64] = accr[ib][ob][j];
          dst[(2 * q + 1) * 64] = acci[ib][ob][j];
        }
  }
  __syncthreads();
  if (!mode_ok) return;
  const int per = NP / S;
  for (int q = s * per; q < (s + 1) * per; ++q) {
    float re = 0.f, im = 0.f;
    for (int v = 0; v < S; ++v) {
      re += red[((size_t)v * NP * 2 + 2 * q) * 64 + lane];
      im += red[((size_t)v * NP * 2 + 2 * q + 1) * 64 + lane];
    }
    const int j = q & 3, ob = (q >> 2) & 3, ib = q >> 4;
    const int i = i0 + 4 * ib + j, o = o0 + 4 * nn + ob;
    if (i < Ci && o < Co) store_pair<DT>(a.dw, 2 * (((size_t)mode * Ci + i) * Co + o), sc * re, sc * im);
  }
}

int gradw_pick_ib(int B, int Ci, int Co, int K) {
  // widest input-channel tile that still leaves >= 1024 waves
  (void)B;
  const long tiles_k = (K + 15) / 16, tiles_o = (Co + 15) / 16;
  for (int ib = 4; ib > 1; ib >>= 1) {
    if (2 * ib >= Ci) continue;  // a narrower tile already covers the channels
    const long waves = tiles_k * tiles_o * ((Ci + 4 * ib - 1) / (4 * ib));
    if (waves >= 1024) return ib;
  }
  return 1;
}

int gradw_pick_split(int B, int Ci, int Co, int K, int ib) {
  // waves per workgroup sharing one tile: enough waves to fill the chip, at
  // least four batch rows per wave
  const long waves = (long)((K + 15) / 16) * ((Co + 15) / 16) * ((Ci + 4 * ib - 1) / (4 * ib));
  int S = 1;
  while (waves * S < 2048 && S < 8 && B >= 8 * S) S *= 2;
  return S;
}

size_t gradw_lds_bytes(int ib, int S) { return S > 1 ? (size_t)S * ib * 32 * 64 * sizeof(float) : 0; }

template <int IB>
static const void *gradw_kernel(int dtype) {
  switch (dtype) {
    case DT_F32: return (const void *)fno_grad_w<IB, DT_F32>;
    case DT_F16: return (const void *)fno_grad_w<IB, DT_F16>;
    case DT_BF16: return (const void *)fno_grad_w<IB, DT_BF16>;
  }
  return nullptr;
}

static const void *gradw_kernel(int ib, int dtype) {
  return ib == 4 ? gradw_kernel<4>(dtype) : ib == 2 ? gradw_kernel<2>(dtype) : gradw_kernel<1>(dtype);
}

hipError_t gradw_prepare(int ib, int dtype, size_t lds) {
  const void *k = gradw_kernel(ib, dtype);
  if (!k) return hipErrorInvalidValue;
  return hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

hipError_t launch_grad_w(const GradWArgs &a, int ib, int S, int dtype, hipStream_t s) {
  const void *k = gradw_kernel(ib, dtype);
  if (!k) return hipErrorInvalidValue;
  const long gy = (a.Ci + 4 * ib - 1) / (4 * ib), gz = (a.Co + 15) / 16;
  if (gy > 65535 || gz > 65535) return hipErrorInvalidValue;
  dim3 grid((a.K + 15) / 16, (unsigned)gy, (unsigned)gz);
  void *args[] = {(void *)&a};
  return hipLaunchKernel(k, grid, dim3(64 * S), args, gradw_lds_bytes(ib, S), s);
}

}  // namespace fno
