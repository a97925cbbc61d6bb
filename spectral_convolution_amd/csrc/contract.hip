// contract.hip - the per-mode complex channel contraction on MFMA.
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

#include "common.hpp"

namespace fno {

template <int DT>
__device__ __forceinline__ void load_w4(const void *w, size_t idx, int nvalid, float (&re)[4], float (&im)[4]) {
  if (nvalid >= 4) {
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
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t < nvalid) {
        const float2 v = load_pair<DT>(w, 2 * (idx + t));
        re[t] = v.x;
        im[t] = v.y;
      } else {
        re[t] = 0.f;
        im[t] = 0.f;
      }
    }
  }
}

template <int BB, int DT>
__global__ __launch_bounds__(64) void fno_contract(ContractArgs a) {
  const int lane = threadIdx.x;
  const int blk = lane >> 2, nn = lane & 3;
  const int K = a.K, Ci = a.Ci, Co = a.Co, B = a.B;
  const int mode = blockIdx.x * 16 + blk;
  const int b0 = blockIdx.y * 4 * BB;
  const int o0 = blockIdx.z * 16;
  const bool mode_ok = mode < K;
  const int ol = o0 + 4 * nn;                   // first of this lane's 4 output channels
  const int nw = mode_ok ? min(4, max(0, Co - ol)) : 0;
  const bool vec = (Co & 3) == 0;

  v4f accr[BB][4], acci[BB][4];
#pragma unroll
  for (int bb = 0; bb < BB; ++bb)
#pragma unroll
    for (int ob = 0; ob < 4; ++ob) {
      accr[bb][ob] = v4f{0.f, 0.f, 0.f, 0.f};
      acci[bb][ob] = v4f{0.f, 0.f, 0.f, 0.f};
    }

  for (int i = 0; i < Ci; ++i) {
    float ar[BB], ai[BB], an[BB];
#pragma unroll
    for (int bb = 0; bb < BB; ++bb) {
      const int b = b0 + 4 * bb + nn;
      float2 xv = make_float2(0.f, 0.f);
      if (mode_ok && b < B) xv = a.xh[((size_t)b * Ci + i) * K + mode];
      ar[bb] = xv.x;
      ai[bb] = xv.y;
      an[bb] = -xv.y;
    }
    float wr[4], wi[4];
    const size_t widx = ((size_t)mode * Ci + i) * Co + ol;
    if (vec) {
      load_w4<DT>(a.w, widx, nw, wr, wi);
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (t < nw) {
          const float2 v = load_pair<DT>(a.w, 2 * (widx + t));
          wr[t] = v.x;
          wi[t] = v.y;
        } else {
          wr[t] = 0.f;
          wi[t] = 0.f;
        }
      }
    }
#pragma unroll
    for (int bb = 0; bb < BB; ++bb)
#pragma unroll
      for (int ob = 0; ob < 4; ++ob) {
        accr[bb][ob] = __builtin_amdgcn_mfma_f32_4x4x1f32(ar[bb], wr[ob], accr[bb][ob], 0, 0, 0);
        accr[bb][ob] = __builtin_amdgcn_mfma_f32_4x4x1f32(an[bb], wi[ob], accr[bb][ob], 0, 0, 0);
        acci[bb][ob] = __builtin_amdgcn_mfma_f32_4x4x1f32(ar[bb], wi[ob], acci[bb][ob], 0, 0, 0);
        acci[bb][ob] = __builtin_amdgcn_mfma_f32_4x4x1f32(ai[bb], wr[ob], acci[bb][ob], 0, 0, 0);
      }
  }

  // accumulator register j of lane l holds block l/4, row j, column l%4
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
}

int contract_pick_bb(int B, int Co, int K) {
  // widest batch tile that still leaves >= 1024 waves for the 256 CUs
  const long tiles_k = (K + 15) / 16, tiles_o = (Co + 15) / 16;
  for (int bb = 4; bb > 1; bb >>= 1) {
    if (2 * bb >= B) continue;  // a narrower tile already covers the batch
    const long waves = tiles_k * tiles_o * ((B + 4 * bb - 1) / (4 * bb));
    if (waves >= 1024) return bb;
  }
  return 1;
}

template <int BB>
static const void *contract_kernel(int dtype) {
  switch (dtype) {
    case DT_F32: return (const void *)fno_contract<BB, DT_F32>;
    case DT_F16: return (const void *)fno_contract<BB, DT_F16>;
    case DT_BF16: return (const void *)fno_contract<BB, DT_BF16>;
  }
  return nullptr;
}

hipError_t launch_contract(const ContractArgs &a, int bb, int dtype, hipStream_t s) {
  const void *k = bb == 4 ? contract_kernel<4>(dtype) : bb == 2 ? contract_kernel<2>(dtype) : contract_kernel<1>(dtype);
  if (!k) return hipErrorInvalidValue;
  dim3 grid((a.K + 15) / 16, (a.B + 4 * bb - 1) / (4 * bb), (a.Co + 15) / 16);
  void *args[] = {(void *)&a};
  return hipLaunchKernel(k, grid, dim3(64), args, 0, s);
}

}  // namespace fno
