// fused.hip - the whole 2D layer as one persistent launch.
//
// The TurboFNO write-up (section 3.4) runs FFT -> GEMM -> iFFT as one fused
// kernel, and its section 5.2 measures the three-kernel split as the slower
// mode. A tile-local fusion cannot work here: every retained mode of a plane
// depends on every pixel of the plane, the contraction of a mode needs every
// input channel of that mode, and the inverse of a plane needs every
// contracted mode. So one launch runs three phases over the same persistent
// grid and joins them with two grid-wide barriers:
//
//   phase F  forward plane transforms (x -> spectra)       | barrier
//   phase C  per-mode contraction (spectra -> spectra)     | barrier
//   phase I  inverse plane transforms (spectra -> y)
//
// Every workgroup of the grid must be resident at once for the barriers to
// complete, so the kernel is launched cooperatively (the runtime refuses a
// grid that cannot be co-resident) with at most the occupancy-derived number
// of workgroups. Each barrier's wait is bounded: a workgroup that has polled
// `spin` times gives up, sets the plan's error word and carries on, so a
// broken grid ends with an error report instead of a hang.
//
// The phases run the same device bodies as the stand-alone kernels, on
// 256-thread workgroups: the VALU plane transforms, or the matrix-core ones
// with four waves and one R column tile per wave; the fp32-matrix-core
// contraction with its input channels split over the four waves.

#include "contract.hpp"
#include "plane_mfma.hpp"
#include "plane_valu.hpp"

#include <algorithm>

namespace fno {

constexpr int kFusedThreads = 256;

// Sense-reversing barrier over all workgroups of the grid. `count` returns
// to zero after every completed barrier and `gen` only grows, so the state
// needs no reset between launches (and a replayed launch sees a consistent
// state). Cross-XCD visibility: after the workgroup barrier (every wave's
// stores done) one thread fences at agent scope before arriving, which writes
// the XCD's L2 back to memory every XCD reads from, and again after leaving,
// which drops stale cached lines of the CU and the XCD; the counter and the
// generation word are agent-scope atomics on separate 128-byte lines, so the
// polls of waiting workgroups do not contend with the arrivals. Measured on
// the 128x128 fp32 layer at batch 16: a fence in every wave instead of one per
// workgroup took the launch from 100 to 141 us; the two words on one line
// instead of two, from 63 to 82 us (plain launches in both cases).
__device__ __forceinline__ bool grid_sync(FusedBarrier *bar, unsigned nblocks, unsigned spin, int *ok_lds) {
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    int ok = 1;
    const unsigned g = __hip_atomic_load(&bar->gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned prev = __hip_atomic_fetch_add(&bar->count, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (prev + 1 == nblocks) {
      __hip_atomic_store(&bar->count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(&bar->gen, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      unsigned n = 0;
      while (__hip_atomic_load(&bar->gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == g) {
        if (++n > spin) {
          ok = 0;
          __hip_atomic_store(&bar->err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    __threadfence();
    *ok_lds = ok;
  }
  __syncthreads();
  return *ok_lds != 0;
}

// phase C: the contraction's (16-mode, 4-row, 16-channel) tiles dealt to
// the workgroups round-robin, the four waves splitting the input channels
template <int DT, bool VEC>
__device__ __forceinline__ void fused_contract(const ContractArgs &c, float *red) {
  const int tx = (c.K + 15) / 16, ty = (c.B + 3) / 4, tz = (c.Co + 15) / 16;
  const int nt = tx * ty * tz;
  for (int t = blockIdx.x; t < nt; t += gridDim.x) {
    const int bz = t % tz, r = t / tz, by = r % ty, bx = r / ty;
    contract_tile<1, DT, VEC>(c, bx, by, bz, kFusedThreads / 64, red);
    __syncthreads();  // red is rewritten by the next tile
  }
}

// VALU planes (MP: pruning size of the register FFTs)
template <int MP, int DT, bool VEC>
__global__ __launch_bounds__(kFusedThreads) void fno_layer_fused(FusedValuArgs a) {
  extern __shared__ u32x4 lds[];
  __shared__ int ok;
  float2 *sm = reinterpret_cast<float2 *>(lds);
  const int nf = (a.fwd.nplanes + a.fwd.ppw - 1) / a.fwd.ppw;
  for (int b = blockIdx.x; b < nf; b += gridDim.x) {
    fwd_plane_block<MP, DT>(a.fwd, b, sm);
    __syncthreads();
  }
  grid_sync(a.bar, a.nbar, a.spin, &ok);
  fused_contract<DT, VEC>(a.ctr, reinterpret_cast<float *>(lds));
  grid_sync(a.bar, a.nbar, a.spin, &ok);
  const int ni = (a.inv.nplanes + a.inv.ppw - 1) / a.inv.ppw;
  for (int b = blockIdx.x; b < ni; b += gridDim.x) {
    inv_plane_block<MP, DT>(a.inv, b, sm);
    __syncthreads();
  }
}

// matrix-core planes (KB = W / 32; at most 16 kx per corner and 16 ky)
template <int DT, int KB, bool VEC>
__global__ __launch_bounds__(kFusedThreads) void fno_layer_fused_mx(FusedMxArgs a) {
  extern __shared__ u32x4 lds[];
  __shared__ int ok;
  fwd_mx_run<DT, KB, 1, kFusedThreads / 64, false>(a.fwd, blockIdx.x, gridDim.x, lds);
  grid_sync(a.bar, a.nbar, a.spin, &ok);
  fused_contract<DT, VEC>(a.ctr, reinterpret_cast<float *>(lds));
  grid_sync(a.bar, a.nbar, a.spin, &ok);
  inv_mx_run<DT, KB, true>(a.inv, blockIdx.x, gridDim.x, lds);
}

// --------------------------------------------------------------- launchers

template <int DT, bool VEC>
static const void *valu_kernel_mp(int MP) {
  switch (MP) {
    case 4: return (const void *)fno_layer_fused<4, DT, VEC>;
    case 8: return (const void *)fno_layer_fused<8, DT, VEC>;
    case 16: return (const void *)fno_layer_fused<16, DT, VEC>;
  }
  return nullptr;
}

template <int DT, bool VEC>
static const void *mx_kernel_w(int W) {
  switch (W) {
    case 64: return (const void *)fno_layer_fused_mx<DT, 2, VEC>;
    case 128: return (const void *)fno_layer_fused_mx<DT, 4, VEC>;
  }
  return nullptr;
}

template <bool VEC>
static const void *fused_kernel_v(const FusedShape &f) {
  if (f.mx) {
    switch (f.dtype) {
      case DT_F32: return mx_kernel_w<DT_F32, VEC>(f.W);
      case DT_F16: return mx_kernel_w<DT_F16, VEC>(f.W);
      case DT_BF16: return mx_kernel_w<DT_BF16, VEC>(f.W);
    }
    return nullptr;
  }
  switch (f.dtype) {
    case DT_F32: return valu_kernel_mp<DT_F32, VEC>(f.MP);
    case DT_F16: return valu_kernel_mp<DT_F16, VEC>(f.MP);
    case DT_BF16: return valu_kernel_mp<DT_BF16, VEC>(f.MP);
  }
  return nullptr;
}

static const void *fused_kernel(const FusedShape &f) {
  return (f.Co & 3) == 0 ? fused_kernel_v<true>(f) : fused_kernel_v<false>(f);
}

bool fused_supported(const FusedShape &f) {
  if (f.mx) return (f.W == 64 || f.W == 128) && f.m1 <= 16 && f.m2 <= 16;
  return f.MP == 4 || f.MP == 8 || f.MP == 16;
}

size_t fused_lds_bytes(const FusedShape &f, size_t lds_fwd, size_t lds_inv) {
  const size_t ctr = contract_lds_bytes(1, kFusedThreads / 64);
  return std::max(std::max(lds_fwd, lds_inv), ctr);
}

hipError_t fused_prepare(const FusedShape &f, size_t lds, int device, int *grid) {
  const void *k = fused_kernel(f);
  if (!k) return hipErrorInvalidValue;
  hipError_t e = raise_lds_cap(k, lds);
  int per_cu = 0, ncu = 0, coop = 0;
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kFusedThreads, lds);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, device);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, device);
  if (e != hipSuccess) return e;
  if (!coop || per_cu < 1 || ncu < 1) return hipErrorNotSupported;
  *grid = per_cu * ncu;
  return hipSuccess;
}

hipError_t launch_layer_fused(const FusedShape &f, const void *args, int grid, size_t lds, hipStream_t s) {
  FNO_BOUNDS(check_layer_fused(f, args, grid, lds);)
  const void *k = fused_kernel(f);
  if (!k || grid < 1) return hipErrorInvalidValue;
  void *kargs[] = {const_cast<void *>(args)};
  return hipLaunchCooperativeKernel(k, dim3(grid), dim3(kFusedThreads), kargs, (unsigned)lds, s);
}

}  // namespace fno
