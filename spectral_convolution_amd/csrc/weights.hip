// weights.hip - repacking spectral weights between the layer's own layout and
// the two layouts a PyTorch FNO module keeps them in.
//
// The TurboFNO write-up (section 2.2, the contraction's learnable weight of
// shape (modes_x, modes_y, in_ch, out_ch); section 4.3, the autograd Function
// that takes it as weight_real and weight_imag) stores the weight split into
// real and imaginary tensors with the modes first. The common FNO module
// instead keeps one complex tensor per spectrum corner, channels first:
// [Ci][Co][m1][m2] for the low and the high kx corner (3D: [Ci][Co][m1][m2][m3]
// for the corners (lo, lo), (hi, lo), (lo, hi), (hi, hi) in kx, ky). The layer
// takes w [modes][Ci][Co][re, im] (modes in spectrum order, the low corner
// first along each cornered axis). These kernels only move elements: no
// arithmetic touches a value, so every layout round-trips bit for bit.

#include "common.hpp"

namespace fno {

// Source index in the corner layout of mode k (the layer's spectrum order).
__device__ __forceinline__ long corner_index(const WeightsArgs &a, long k, int i, int o) {
  int c, r;
  if (a.ndim == 2) {
    const int ax = (int)(k / a.m2), ky = (int)(k % a.m2);
    const int cx = ax >= a.m1;
    c = cx;
    r = (ax - cx * a.m1) * a.m2 + ky;
  } else {
    const int kz = (int)(k % a.m3);
    const long t = k / a.m3;
    const int ay = (int)(t % (2 * a.m2)), ax = (int)(t / (2 * a.m2));
    const int cx = ax >= a.m1, cy = ay >= a.m2;
    c = cx + 2 * cy;
    r = ((ax - cx * a.m1) * a.m2 + (ay - cy * a.m2)) * a.m3 + kz;
  }
  return (((long)c * a.Ci + i) * a.Co + o) * a.mc + r;
}

// P: one (re, im) pair; S: one real. unpack = false copies the user's layout
// into w, true copies w back out.
template <typename P, typename S>
__global__ __launch_bounds__(256) void fno_weights_repack(WeightsArgs a) {
  const long cico = (long)a.Ci * a.Co;
  for (long j = blockIdx.x * 256L + threadIdx.x; j < a.n; j += (long)gridDim.x * 256) {
    P *w = (P *)a.w + j;
    if (a.layout == W_SPLIT) {
      S *re = (S *)a.re + j, *im = (S *)a.im + j;
      if (!a.unpack) {
        P v;
        v.x = *re;
        v.y = *im;
        *w = v;
      } else {
        const P v = *w;
        *re = v.x;
        *im = v.y;
      }
    } else {
      const long k = j / cico, io = j - k * cico;
      P *src = (P *)a.re + corner_index(a, k, (int)(io / a.Co), (int)(io % a.Co));
      if (!a.unpack)
        *w = *src;
      else
        *src = *w;
    }
  }
}

struct pair16 {
  uint16_t x, y;
};

hipError_t launch_weights_repack(const WeightsArgs &a, int dtype, hipStream_t s) {
  FNO_BOUNDS(check_weights_repack(a, dtype);)
  if (a.n < 1) return hipSuccess;
  const long blocks = (a.n + 255) / 256;
  const dim3 grid((unsigned)(blocks < 65536 ? blocks : 65536));
  if (dtype == DT_F32)
    hipLaunchKernelGGL((fno_weights_repack<uint2, uint32_t>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((fno_weights_repack<pair16, uint16_t>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace fno
