// contract.hip - the per-mode contraction on fp32 matrix cores as a
// stand-alone kernel (one output tile per workgroup), the backward's adjoint
// contraction that reads W in its forward layout, and their launchers.

#include "contract.hpp"

namespace fno {

template <int BB, int DT, bool VEC>
__global__ __launch_bounds__(512) void fno_contract(ContractArgs a) {
  extern __shared__ float red[];
  contract_tile<BB, DT, VEC>(a, blockIdx.x, blockIdx.y, blockIdx.z, blockDim.x >> 6, red);
}

// Adjoint contraction reading W in its forward layout (fp32 storage); one
// wave per 16 modes x 4 BB batch rows x 16 output channels, the reduction
// split over the S waves of a workgroup, each wave with its own LDS region.
template <int BB>
__global__ __launch_bounds__(512) void fno_contract_adj(ContractArgs a) {
  extern __shared__ float2 stg[];
  contract_tile_adj<BB>(a, blockIdx.x, blockIdx.y, blockIdx.z, blockDim.x >> 6, stg);
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

// The adjoint straight from W: fp32 storage, an even number of reduction
// channels (the layer's c_out), and batch tiles of 4 rows (bb = 1). Plans
// whose adjoint takes wider batch tiles keep the transposed copy: this
// kernel would read W once per 4 batch rows.
bool contract_adj_supported(int dtype, int c_out, int bb) {
  return dtype == DT_F32 && c_out >= 2 && c_out % 2 == 0 && bb == 1;
}

// per wave: its staging region, or its partial sums when larger
static size_t adj_wave_bytes(int bb) {
  const size_t stage = (size_t)AdjL::WAVE * sizeof(float2), red = (size_t)bb * 16 * 2 * 64 * sizeof(float);
  return stage > red ? stage : red;
}

size_t contract_adj_lds_bytes(int bb, int S) { return (size_t)S * adj_wave_bytes(bb); }

static const void *contract_adj_kernel(int bb) { return bb == 1 ? (const void *)fno_contract_adj<1> : nullptr; }

hipError_t contract_adj_prepare(int bb, int S) {
  const void *k = contract_adj_kernel(bb);
  return k ? raise_lds_cap(k, contract_adj_lds_bytes(bb, S)) : hipErrorInvalidValue;
}

hipError_t launch_contract_adj(const ContractArgs &a, int bb, int S, hipStream_t s) {
  FNO_BOUNDS(check_contract_adj(a, bb, S, adj_wave_bytes(bb), AdjL::WAVE * sizeof(float2));)
  const void *k = contract_adj_kernel(bb);
  if (!k || (S != 1 && S != 2 && S != 4 && S != 8) || a.Ci < 2 || a.Ci % 2) return hipErrorInvalidValue;
  dim3 grid((a.K + 15) / 16, (a.B + 4 * bb - 1) / (4 * bb), (a.Co + 15) / 16);
  void *args[] = {(void *)&a};
  return hipLaunchKernel(k, grid, dim3(64 * S), args, contract_adj_lds_bytes(bb, S), s);
}

}  // namespace fno
