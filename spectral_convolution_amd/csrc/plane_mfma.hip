// plane_mfma.hip - the matrix-core plane transforms as stand-alone
// persistent kernels (one workgroup per resident slot), and their launchers.

#include "plane_mfma.hpp"

namespace fno {

template <int DT, int KB, int CPW, int NW, bool TW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void fno_fwd_plane_mx(PlaneMxFwdArgs a) {
  extern __shared__ u32x4 lds[];
  fwd_mx_run<DT, KB, CPW, NW, TW>(a, blockIdx.x, gridDim.x, lds);
}

template <int DT, int KB, bool SM, bool HX>
__global__ __launch_bounds__(kFT) __attribute__((amdgpu_waves_per_eu(SM ? 3 : 2))) void fno_inv_plane_mx(PlaneMxInvArgs a) {
  extern __shared__ u32x4 lds[];
  inv_mx_run<DT, KB, SM, HX>(a, blockIdx.x, gridDim.x, lds);
}

// The inverse column stage alone (fp16 / bf16): Z rows to a.zg for the FNO
// block's row-stage kernel. The row-stage width does not enter the column
// stage, so one instantiation (the 64-wide layout) serves every W.
template <int DT, bool SM, bool HX>
__global__ __launch_bounds__(kFT) __attribute__((amdgpu_waves_per_eu(SM ? 3 : 2))) void fno_inv_cols_mx(PlaneMxInvArgs a) {
  extern __shared__ u32x4 lds[];
  inv_mx_run<DT, 2, SM, HX, true>(a, blockIdx.x, gridDim.x, lds);
}

// --------------------------------------------------------------- launchers

bool mx_supported(int H, int W, int m1, int m2, int dtype) {
  // fp32 carries hi + lo twiddle parts in registers: narrower planes, fewer modes
  const int wmax = dtype == DT_F32 ? 128 : 256, m1max = 32;
  return (dtype == DT_F16 || dtype == DT_BF16 || dtype == DT_F32) && H >= kRows && H <= 256 && W >= 64 &&
         W <= wmax && m1 <= m1max && m2 <= 32 && 2 * m1 <= H;
}

int mx_ntiles(int m2) { return m2 <= 8 ? 1 : m2 <= 16 ? 2 : 4; }

size_t mx_fwd_lds_bytes(int H, int W, int dtype) {
  const size_t np = dtype == DT_F32 ? 2 : 1;
  return 2 * np * kRows * (W / 8 + 2) * 16 + 2 * np * 32 * kRBP * 2 + (size_t)H * 8 + 16 * 4;
}

static bool inv_small(int m1, int m2) { return m1 <= 16 && m2 <= 16; }

template <bool SM>
static size_t inv_lds(int H, int W, int dtype) {
  using G = InvGeom<SM>;
  const size_t np = dtype == DT_F32 ? 2 : 1, es = dtype == DT_F32 ? 4 : 2;
  return (size_t)kRows * (W * es / 16 + 1) * 16 + np * ((size_t)G::YR * G::YP + (size_t)kRows * G::ZP) * 2 +
         (size_t)H * 8 + 64;
}

size_t mx_inv_lds_bytes(int H, int W, int m1, int m2, int dtype) {
  return inv_small(m1, m2) ? inv_lds<true>(H, W, dtype) : inv_lds<false>(H, W, dtype);
}

// Forward workgroup shape: 8 waves where one workgroup per CU is all the
// LDS or the m-tiles allow (W = 256, split-operand W = 128, more than four
// m-tiles), else 4; two R c-tiles per wave only if every wave still gets a
// row-product job (4 row blocks x c-tile groups >= waves).
struct FwdCfg {
  int nw, cpw;
};

static FwdCfg fwd_cfg(int W, int m1, int m2, int dtype) {
  const int kb = W / 32, mt = (m1 + 3) / 4, nt = mx_ntiles(m2);
  const bool sp = dtype == DT_F32;
  const int nw = (kb == 8 || (sp && kb == 4) || mt > 4) ? 8 : 4;
  return {nw, nt >= 2 && 2 * nt >= nw ? 2 : 1};
}

int mx_fwd_waves(int W, int m1, int m2, int dtype) { return fwd_cfg(W, m1, m2, dtype).nw; }

template <int DT, int KB, bool TW>
static const void *mx_fwd_kernel(FwdCfg c) {
  if (c.nw == 8)
    return c.cpw == 2 ? (const void *)fno_fwd_plane_mx<DT, KB, 2, 8, TW> : (const void *)fno_fwd_plane_mx<DT, KB, 1, 8, TW>;
  if constexpr (KB == 8 || (DT == DT_F32 && KB == 4)) return nullptr;  // always 8 waves
  else return c.cpw == 2 ? (const void *)fno_fwd_plane_mx<DT, KB, 2, 4, TW> : (const void *)fno_fwd_plane_mx<DT, KB, 1, 4, TW>;
}

template <int DT, int KB, bool HX>
static const void *mx_inv_kernel(bool small) {
  return small ? (const void *)fno_inv_plane_mx<DT, KB, true, HX> : (const void *)fno_inv_plane_mx<DT, KB, false, HX>;
}

// half: the inverse kernel that reads the half exchange (fp16 / bf16 only)
template <int DT, int KB>
static const void *mx_kernel_kb(bool fwd, FwdCfg c, bool small, bool two, bool half) {
  if (!fwd) {
    if constexpr (DT == DT_F32) return half ? nullptr : mx_inv_kernel<DT, KB, false>(small);
    else return half ? mx_inv_kernel<DT, KB, true>(small) : mx_inv_kernel<DT, KB, false>(small);
  }
  return two ? mx_fwd_kernel<DT, KB, true>(c) : mx_fwd_kernel<DT, KB, false>(c);
}

template <int DT>
static const void *mx_kernel_dt(bool fwd, int W, FwdCfg c, bool small, bool two, bool half) {
  switch (W) {
    case 64: return mx_kernel_kb<DT, 2>(fwd, c, small, two, half);
    case 128: return mx_kernel_kb<DT, 4>(fwd, c, small, two, half);
    case 256:
      if constexpr (DT == DT_F32) return nullptr;
      else return mx_kernel_kb<DT, 8>(fwd, c, small, two, half);
  }
  return nullptr;
}

// two: the forward kernel that takes two plane sets (fwd only); half: the
// inverse kernel that reads the half exchange (inverse only)
static const void *mx_kernel(bool fwd, int W, int m1, int m2, int dtype, bool two = false, bool half = false) {
  const FwdCfg c = fwd_cfg(W, m1, m2, dtype);
  const bool small = inv_small(m1, m2);
  if (dtype == DT_F16) return mx_kernel_dt<DT_F16>(fwd, W, c, small, two, half);
  if (dtype == DT_BF16) return mx_kernel_dt<DT_BF16>(fwd, W, c, small, two, half);
  if (dtype == DT_F32) return mx_kernel_dt<DT_F32>(fwd, W, c, small, two, half);
  return nullptr;
}

hipError_t mx_prepare(bool fwd, int W, int m1, int m2, int dtype, size_t lds, bool two) {
  const void *k = mx_kernel(fwd, W, m1, m2, dtype, two);
  if (!k) return hipErrorInvalidValue;
  hipError_t e = raise_lds_cap(k, lds);
  // the half-exchange inverse shares the LDS size of the fp32-exchange one
  if (e == hipSuccess && !fwd && dtype != DT_F32) e = raise_lds_cap(mx_kernel(false, W, m1, m2, dtype, false, true), lds);
  return e;
}

// workgroups of a persistent plane kernel: as many as are resident at once
// on the device (never more than planes)
hipError_t mx_grid(bool fwd, int W, int m1, int m2, int dtype, size_t lds, int device, int nplanes, int *grid,
                   bool two) {
  const void *k = mx_kernel(fwd, W, m1, m2, dtype, two);
  if (!k) return hipErrorInvalidValue;
  int per_cu = 0, ncu = 0;
  const int threads = fwd ? fwd_cfg(W, m1, m2, dtype).nw * 64 : kFT;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, threads, lds);
  if (e == hipSuccess && !fwd && dtype != DT_F32) {  // the half-exchange variant too: the smaller of the two
    int per_cu_h = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_h, mx_kernel(false, W, m1, m2, dtype, false, true),
                                                     threads, lds);
    per_cu = per_cu_h < per_cu ? per_cu_h : per_cu;
  }
  if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) return e;
  long g = (long)(per_cu > 0 ? per_cu : 1) * (ncu > 0 ? ncu : 1);
  *grid = (int)(g < nplanes ? g : nplanes);
  return hipSuccess;
}

hipError_t launch_plane_mx_fwd(const PlaneMxFwdArgs &a, int grid, int dtype, size_t lds, hipStream_t s, bool two) {
  FNO_BOUNDS(check_plane_mx_fwd(a, grid, dtype, lds, two);)
  const void *k = mx_kernel(true, a.W, a.m1, a.m2, dtype, two);
  if (!k || grid < 1) return hipErrorInvalidValue;
  void *args[] = {(void *)&a};
  return hipLaunchKernel(k, dim3(grid), dim3(fwd_cfg(a.W, a.m1, a.m2, dtype).nw * 64), args, lds, s);
}

hipError_t launch_plane_mx_inv(const PlaneMxInvArgs &a, int grid, int dtype, size_t lds, hipStream_t s) {
  FNO_BOUNDS(check_plane_mx_inv(a, grid, dtype, lds, false);)
  const void *k = mx_kernel(false, a.W, a.m1, a.m2, dtype, false, a.in16 != nullptr);
  if (!k || grid < 1) return hipErrorInvalidValue;
  void *args[] = {(void *)&a};
  return hipLaunchKernel(k, dim3(grid), dim3(kFT), args, lds, s);
}

// column stage only
template <int DT, bool HX>
static const void *cols_kernel_dt(bool small) {
  return small ? (const void *)fno_inv_cols_mx<DT, true, HX> : (const void *)fno_inv_cols_mx<DT, false, HX>;
}

static const void *cols_kernel(int m1, int m2, int dtype, bool half) {
  const bool small = inv_small(m1, m2);
  if (dtype == DT_F16) return half ? cols_kernel_dt<DT_F16, true>(small) : cols_kernel_dt<DT_F16, false>(small);
  if (dtype == DT_BF16) return half ? cols_kernel_dt<DT_BF16, true>(small) : cols_kernel_dt<DT_BF16, false>(small);
  return nullptr;
}

hipError_t mx_cols_prepare(int m1, int m2, int dtype, size_t lds, int device, int nplanes, int *grid) {
  int per_cu = 1 << 20, ncu = 0;
  for (bool half : {false, true}) {
    const void *k = cols_kernel(m1, m2, dtype, half);
    if (!k) return hipErrorInvalidValue;
    hipError_t e = raise_lds_cap(k, lds);
    int pc = 0;
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&pc, k, kFT, lds);
    if (e != hipSuccess) return e;
    per_cu = pc < per_cu ? pc : per_cu;
  }
  hipError_t e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) return e;
  const long g = (long)(per_cu > 0 ? per_cu : 1) * (ncu > 0 ? ncu : 1);
  *grid = (int)(g < nplanes ? g : nplanes);
  return hipSuccess;
}

hipError_t launch_plane_mx_cols(const PlaneMxInvArgs &a, int grid, int dtype, size_t lds, hipStream_t s) {
  FNO_BOUNDS(check_plane_mx_inv(a, grid, dtype, lds, true);)
  const void *k = cols_kernel(a.m1, a.m2, dtype, a.in16 != nullptr);
  if (!k || grid < 1 || !a.zg || !a.zexp || a.zco < 1) return hipErrorInvalidValue;
  void *args[] = {(void *)&a};
  return hipLaunchKernel(k, dim3(grid), dim3(kFT), args, lds, s);
}

}  // namespace fno
