// contract.hip - the per-mode contraction on fp32 matrix cores as a
// stand-alone kernel (one output tile per workgroup) and its launcher.

#include "contract.hpp"

namespace fno {

template <int BB, int DT, bool VEC>
__global__ __launch_bounds__(512) void fno_contract(ContractArgs a) {
  extern __shared__ float red[];
  contract_tile<BB, DT, VEC>(a, blockIdx.x, blockIdx.y, blockIdx.z, blockDim.x >> 6, red);
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

template <int BB, bool VEC>
static const void *contract_kernel_v(int dtype) {
  switch (dtype) {
    case DT_F32: return (const void *)fno_contract<BB, DT_F32, VEC>;
    case DT_F16: return (const void *)fno_contract<BB, DT_F16, VEC>;
    case DT_BF16: return (const void *)fno_contract<BB, DT_BF16, VEC>;
  }
  return nullptr;
}

template <int BB>
static const void *contract_kernel(int dtype, int Co) {
  return (Co & 3) == 0 ? contract_kernel_v<BB, true>(dtype) : contract_kernel_v<BB, false>(dtype);
}

int contract_pick_split(int B, int Ci, int Co, int K, int bb) {
  // waves per workgroup sharing one output tile: enough waves in flight to
  // fill the chip, at least two input channels per wave
  const long waves = (long)((K + 15) / 16) * ((Co + 15) / 16) * ((B + 4 * bb - 1) / (4 * bb));
  int S = 1;
  while (waves * S < 2048 && S < 8 && Ci >= 4 * S) S *= 2;
  return S;
}

size_t contract_lds_bytes(int bb, int S) { return S > 1 ? (size_t)S * bb * 32 * 64 * sizeof(float) : 0; }

hipError_t contract_prepare(int bb, int dtype, int Co, size_t lds) {
  const void *k = bb == 4 ? contract_kernel<4>(dtype, Co) : bb == 2 ? contract_kernel<2>(dtype, Co) : contract_kernel<1>(dtype, Co);
  if (!k) return hipErrorInvalidValue;
  return raise_lds_cap(k, lds);
}

hipError_t launch_contract(const ContractArgs &a, int bb, int S, int dtype, hipStream_t s) {
  FNO_BOUNDS(check_contract(a, dtype, false);)
  const void *k = bb == 4 ? contract_kernel<4>(dtype, a.Co) : bb == 2 ? contract_kernel<2>(dtype, a.Co)
                                                           : contract_kernel<1>(dtype, a.Co);
  if (!k) return hipErrorInvalidValue;
  dim3 grid((a.K + 15) / 16, (a.B + 4 * bb - 1) / (4 * bb), (a.Co + 15) / 16);
  void *args[] = {(void *)&a};
  return hipLaunchKernel(k, grid, dim3(64 * S), args, contract_lds_bytes(bb, S), s);
}

}  // namespace fno
