// plane_kernels.hip - pruned forward / inverse 2D transforms of real planes.
//
// A 256-thread workgroup handles `ppw` whole planes (more than one when the
// planes are small). The transforms keep only the retained low-frequency
// modes of the FNO layer (TurboFNO write-up, sections 2.2 and 2.3: corners
// in kx, half spectrum in ky) and never form the full spectrum.
//
// Pruning by decimation: with MP = next_pow2(max mode count) and P = N / MP,
// sample n of a length-N axis is split as n = r + P q (residue r < P,
// q < MP). Forward, an MP-point DFT over q of every residue gives D_r[j];
// a retained output k is sum_r w^(r k) D_r[k mod MP], w = exp(-2 pi i / N).
// Inverse (input pruned), the retained inputs are pre-multiplied per residue
// and one MP-point inverse DFT per residue yields the strided outputs
// n = r + P q directly.
//
// Row (contiguous, real) axis: chunks of rows are copied between global
// memory and LDS with coalesced 16-byte accesses (one wave instruction moves
// 1 KiB of consecutive bytes); in LDS a thread takes two adjacent residues of
// one row and packs them as the real and imaginary parts of one complex
// sequence (one complex FFT for two real ones). Forward, the residues'
// weighted sums are added over the T = P/2 threads of a row by a butterfly
// across lanes (DPP quad permutes and row mirrors). Column axis: one thread
// per (column, residue), partial sums reduced the same way. LDS holds the
// row spectra (H x m2 per plane), one staging chunk and the twiddle tables.

#include "plane_valu.hpp"

namespace fno {


// residues per thread along the row axis (two per complex FFT)
int plane_rpt(int MP, int PW) {
  (void)MP;
  (void)PW;
  return 2;
}

// residues per thread in the column stage: lane groups of at most 64
int plane_rc(int H, int MP) {
  const int PH = H / MP;
  return PH > 64 ? PH / 64 : 1;
}

size_t plane_fwd_lds_bytes(int H, int W, int m1, int m2, int MP, int ppw) {
  (void)m1;
  const size_t stage = (size_t)chunk_rows(W, MP) * stage_pitch(W, MP) * sizeof(float);
  return ((size_t)W + H + (size_t)ppw * H * (m2 + 1)) * sizeof(float2) + stage;
}

size_t plane_inv_lds_bytes(int H, int W, int m1, int m2, int MP, int ppw) {
  const size_t stage = (size_t)chunk_rows(W, MP) * stage_pitch(W, MP) * sizeof(float);
  return ((size_t)W + H + (size_t)ppw * (2 * m1 * m2 + (size_t)H * (m2 + 1))) * sizeof(float2) + stage;
}

// planes per workgroup: at least one chunk of rows, within 64 KiB of LDS
int plane_ppw(bool fwd, int H, int W, int m1, int m2, int MP, int nplanes) {
  int ppw = chunk_rows(W, MP) / H;
  if (ppw < 1) ppw = 1;
  if (ppw > nplanes) ppw = nplanes;
  while (ppw > 1 && (fwd ? plane_fwd_lds_bytes(H, W, m1, m2, MP, ppw) : plane_inv_lds_bytes(H, W, m1, m2, MP, ppw)) >
                        64 * 1024)
    ppw >>= 1;
  return ppw;
}

template <int MP, int DT>
__global__ __launch_bounds__(kThreads) void fno_fwd_plane(PlaneFwdArgs a) {
  extern __shared__ float2 smem[];
  fwd_plane_block<MP, DT>(a, blockIdx.x, smem);
}

template <int MP, int DT>
__global__ __launch_bounds__(kThreads) void fno_inv_plane(PlaneInvArgs a) {
  extern __shared__ float2 smem[];
  inv_plane_block<MP, DT>(a, blockIdx.x, smem);
}

// --------------------------------------------------------------- launchers

template <int DT, bool FWD>
static const void *kernel_for(int MP, int rpt) {
  if (rpt != 2) return nullptr;
  switch (MP) {
    case 2: return FWD ? (const void *)fno_fwd_plane<2, DT> : (const void *)fno_inv_plane<2, DT>;
    case 4: return FWD ? (const void *)fno_fwd_plane<4, DT> : (const void *)fno_inv_plane<4, DT>;
    case 8: return FWD ? (const void *)fno_fwd_plane<8, DT> : (const void *)fno_inv_plane<8, DT>;
    case 16: return FWD ? (const void *)fno_fwd_plane<16, DT> : (const void *)fno_inv_plane<16, DT>;
    case 32: return FWD ? (const void *)fno_fwd_plane<32, DT> : (const void *)fno_inv_plane<32, DT>;
  }
  return nullptr;
}

static const void *plane_kernel(bool fwd, int MP, int rpt, int dtype) {
  switch (dtype) {
    case DT_F32: return fwd ? kernel_for<DT_F32, true>(MP, rpt) : kernel_for<DT_F32, false>(MP, rpt);
    case DT_F16: return fwd ? kernel_for<DT_F16, true>(MP, rpt) : kernel_for<DT_F16, false>(MP, rpt);
    case DT_BF16: return fwd ? kernel_for<DT_BF16, true>(MP, rpt) : kernel_for<DT_BF16, false>(MP, rpt);
  }
  return nullptr;
}

hipError_t plane_prepare(bool fwd, int MP, int rpt, int dtype, size_t lds) {
  const void *k = plane_kernel(fwd, MP, rpt, dtype);
  if (!k) return hipErrorInvalidValue;
  return raise_lds_cap(k, lds);
}

hipError_t launch_plane_fwd(const PlaneFwdArgs &a, int MP, int rpt, int dtype, size_t lds, hipStream_t s) {
  FNO_BOUNDS(check_plane_fwd(a, MP, rpt, dtype, lds);)
  const void *k = plane_kernel(true, MP, rpt, dtype);
  if (!k) return hipErrorInvalidValue;
  void *args[] = {(void *)&a};
  return hipLaunchKernel(k, dim3((a.nplanes + a.ppw - 1) / a.ppw), dim3(kThreads), args, lds, s);
}

hipError_t launch_plane_inv(const PlaneInvArgs &a, int MP, int rpt, int dtype, size_t lds, hipStream_t s) {
  FNO_BOUNDS(check_plane_inv(a, MP, rpt, dtype, lds);)
  const void *k = plane_kernel(false, MP, rpt, dtype);
  if (!k) return hipErrorInvalidValue;
  void *args[] = {(void *)&a};
  return hipLaunchKernel(k, dim3((a.nplanes + a.ppw - 1) / a.ppw), dim3(kThreads), args, lds, s);
}

}  // namespace fno
