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
  FNO_BOUNDS(check_conj_transpose(w, wh, K, Ci, Co, dtype);)
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
// Per mode k the weight gradient is a real-form product with the batch as
// the reduction dimension:
//   Re dw[k] = Xr^T Gr + Xi^T Gi,   Im dw[k] = Xr^T Gi + (-Xi)^T Gr
// (X = Xs[.][.][k] as B x Ci, G = Gs[.][.][k] as B x Co). Instruction:
// v_mfma_f32_16x16x4f32 (fp32 operands, fp32 accumulation), one 16 x 16
// (i, o) tile of one mode and four batch rows per instruction.
//
// A workgroup (4 waves) owns MB consecutive modes x CT input x CT output
// channels (16 x 32 x 32, or 8 x 16 x 16 when the large tiles would leave
// most compute units idle) and streams the batch in stages of 4 rows. Each
// stage's spectra rows ([b][i][MB modes] and [b][o][MB modes], 8 * MB
// contiguous bytes each) are loaded with 16-byte accesses one stage ahead
// into registers and stored into LDS per mode as [mode][b][channel]
// (float2), so a fragment read is 16 consecutive channels per lane group.
// Wave w multiplies modes w MB/4 .. (w + 1) MB/4 - 1, all (CT/16)^2 tiles.
// Rows past the batch, channels and modes past their ends load as zeros.

constexpr int kGwT = 256;  // threads per workgroup
constexpr int kGwB = 4;    // batch rows per stage (one MFMA k-step)

template <int MB, int CT>
struct GwShape {
  static constexpr int MW = MB / 4;                  // modes per wave
  static constexpr int NT = CT / 16;                 // 16-wide tiles per channel axis
  static constexpr int P = CT + 1;                   // float2 per batch row of a staged mode (+ pad)
  static constexpr int S = kGwB * P + 1;             // float2 per staged mode (+ pad: stores spread over banks)
  static constexpr int U = kGwB * CT * MB / 2 / kGwT;  // 16-byte units per thread and operand
  static constexpr int PR = MB / 2;                  // mode pairs per row
};

typedef unsigned gw_u32x4 __attribute__((ext_vector_type(4)));

// one stage of one operand: rows (b, c) of MB modes, c fastest, from
// src[b][c][K] (nc channels); unit u = (row, mode pair)
template <int MB, int CT>
__device__ __forceinline__ void gw_fetch(const float2 *src, int nc, int K, int B, int st, int k0, int c0, int tid,
                                         gw_u32x4 (&p)[GwShape<MB, CT>::U]) {
  using G = GwShape<MB, CT>;
#pragma unroll
  for (int v = 0; v < G::U; ++v) {
    const int u = v * kGwT + tid;
    const int row = u / G::PR, pr = u % G::PR;
    const int b = st * kGwB + row / CT, c = c0 + row % CT, mode = k0 + 2 * pr;
    const bool ok = b < B && c < nc && mode < K;
    const gw_u32x4 t = *reinterpret_cast<const gw_u32x4 *>(src + (ok ? ((size_t)b * nc + c) * K + mode : 0));
    p[v] = ok ? t : gw_u32x4{0u, 0u, 0u, 0u};
  }
}

// Half exchange: the spectra as fp16 (re, im) pairs, 4 modes per 16-byte
// unit, plane (b, c) scaled by 2^exp[b][c]; decoded to fp32 on staging.
template <int MB, int CT>
struct GwShape16 {
  static constexpr int N = kGwB * CT * MB / 4;        // 16-byte units of a stage and operand
  static constexpr int U = (N + kGwT - 1) / kGwT;     // per thread (the last pass may be partial)
  static constexpr int QR = MB / 4;                   // mode quads per row
};

template <int MB, int CT>
__device__ __forceinline__ void gw_fetch16(const uint32_t *src, const int *ex, int nc, int K, int B, int st, int k0,
                                           int c0, int tid, gw_u32x4 (&p)[GwShape16<MB, CT>::U],
                                           int (&e)[GwShape16<MB, CT>::U]) {
  using G = GwShape16<MB, CT>;
#pragma unroll
  for (int v = 0; v < G::U; ++v) {
    const int u = v * kGwT + tid;
    const int row = u / G::QR, qr = u % G::QR;
    const int b = st * kGwB + row / CT, c = c0 + row % CT, mode = k0 + 4 * qr;
    const bool ok = u < G::N && b < B && c < nc && mode < K;
    const size_t r = ok ? (size_t)b * nc + c : 0;
    const gw_u32x4 t = *reinterpret_cast<const gw_u32x4 *>(src + (ok ? r * K + mode : 0));
    p[v] = ok ? t : gw_u32x4{0u, 0u, 0u, 0u};
    e[v] = ex[r];
  }
}

template <int MB, int CT>
__device__ __forceinline__ void gw_put16(float2 *stage, int tid, const gw_u32x4 (&p)[GwShape16<MB, CT>::U],
                                         const int (&e)[GwShape16<MB, CT>::U]) {
  using G = GwShape<MB, CT>;
  using H = GwShape16<MB, CT>;
#pragma unroll
  for (int v = 0; v < H::U; ++v) {
    const int u = v * kGwT + tid;
    if (u >= H::N) continue;
    const int row = u / H::QR, qr = u % H::QR;
    const int b = row / CT, c = row % CT;
    const float sc = pow2f(-e[v]);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      // each half converted on its own
      const float re = (float)__builtin_bit_cast(_Float16, (uint16_t)(p[v][t] & 0xffffu)) * sc;
      const float im = (float)__builtin_bit_cast(_Float16, (uint16_t)(p[v][t] >> 16)) * sc;
      stage[(4 * qr + t) * G::S + b * G::P + c] = make_float2(re, im);
    }
  }
}

template <int MB, int CT>
__device__ __forceinline__ void gw_put(float2 *stage, int tid, const gw_u32x4 (&p)[GwShape<MB, CT>::U]) {
  using G = GwShape<MB, CT>;
#pragma unroll
  for (int v = 0; v < G::U; ++v) {
    const int u = v * kGwT + tid;
    const int row = u / G::PR, pr = u % G::PR;
    const int b = row / CT, c = row % CT;
    stage[(2 * pr) * G::S + b * G::P + c] = make_float2(__uint_as_float(p[v][0]), __uint_as_float(p[v][1]));
    stage[(2 * pr + 1) * G::S + b * G::P + c] = make_float2(__uint_as_float(p[v][2]), __uint_as_float(p[v][3]));
  }
}

template <int DT, int MB, int CT, bool HX>
__global__ __launch_bounds__(kGwT) __attribute__((amdgpu_waves_per_eu(2))) void fno_grad_w(GradWArgs a) {
  using G = GwShape<MB, CT>;
  constexpr int MW = G::MW, NT = G::NT;
  __shared__ float2 xs[MB * G::S], gs[MB * G::S];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int K = a.K, Ci = a.Ci, Co = a.Co, B = a.B;
  // workgroups of one mode block are gridDim.x apart: with gridDim.x a
  // multiple of 8 they share an XCD (and its L2), where the second read of
  // each spectra row hits
  const int k0 = blockIdx.x * MB;
  const int nto = (Co + CT - 1) / CT;
  const int i0 = (blockIdx.y / nto) * CT, o0 = (blockIdx.y % nto) * CT;
  const int nst = (B + kGwB - 1) / kGwB;

  v4f accr[MW][NT][NT], acci[MW][NT][NT];
#pragma unroll
  for (int m = 0; m < MW; ++m)
#pragma unroll
    for (int ti = 0; ti < NT; ++ti)
#pragma unroll
      for (int to = 0; to < NT; ++to) {
        accr[m][ti][to] = v4f{0.f, 0.f, 0.f, 0.f};
        acci[m][ti][to] = v4f{0.f, 0.f, 0.f, 0.f};
      }

  constexpr int NU = HX ? GwShape16<MB, CT>::U : G::U;
  gw_u32x4 px[NU], pg[NU];
  int ex[HX ? NU : 1], eg[HX ? NU : 1];
  auto fetch = [&](int st) {
    if constexpr (HX) {
      gw_fetch16<MB, CT>(a.xs16, a.xexp, Ci, K, B, st, k0, i0, tid, px, ex);
      gw_fetch16<MB, CT>(a.gs16, a.gexp, Co, K, B, st, k0, o0, tid, pg, eg);
    } else {
      gw_fetch<MB, CT>(a.xs, Ci, K, B, st, k0, i0, tid, px);
      gw_fetch<MB, CT>(a.gs, Co, K, B, st, k0, o0, tid, pg);
    }
  };
  fetch(0);
  for (int st = 0; st < nst; ++st) {
    if constexpr (HX) {
      gw_put16<MB, CT>(xs, tid, px, ex);
      gw_put16<MB, CT>(gs, tid, pg, eg);
    } else {
      gw_put<MB, CT>(xs, tid, px);
      gw_put<MB, CT>(gs, tid, pg);
    }
    if (st + 1 < nst) fetch(st + 1);
    __syncthreads();
    // fragment of lane l: batch row l / 16, channel 16 t + l % 16
    const int fo = (lane >> 4) * G::P + (lane & 15);
#pragma unroll
    for (int m = 0; m < MW; ++m) {
      const int mm = MW * wv + m;
      float2 x[NT], g[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        x[t] = xs[mm * G::S + fo + 16 * t];
        g[t] = gs[mm * G::S + fo + 16 * t];
      }
#pragma unroll
      for (int ti = 0; ti < NT; ++ti)
#pragma unroll
        for (int to = 0; to < NT; ++to) {
          v4f &cr = accr[m][ti][to], &ci = acci[m][ti][to];
          cr = __builtin_amdgcn_mfma_f32_16x16x4f32(x[ti].x, g[to].x, cr, 0, 0, 0);
          cr = __builtin_amdgcn_mfma_f32_16x16x4f32(x[ti].y, g[to].y, cr, 0, 0, 0);
          ci = __builtin_amdgcn_mfma_f32_16x16x4f32(x[ti].x, g[to].y, ci, 0, 0, 0);
          ci = __builtin_amdgcn_mfma_f32_16x16x4f32(-x[ti].y, g[to].x, ci, 0, 0, 0);
        }
    }
    __syncthreads();
  }

  // accumulator register j of lane l: row 4 (l / 16) + j (input channel),
  // column l % 16 (output channel); 16 lanes store 16 consecutive outputs
#pragma unroll
  for (int m = 0; m < MW; ++m) {
    const int mode = k0 + MW * wv + m;
    if (mode >= K) continue;
    const float sc = a.scale * ((mode % a.mlast) == 0 ? 1.0f : 2.0f);
#pragma unroll
    for (int ti = 0; ti < NT; ++ti)
#pragma unroll
      for (int to = 0; to < NT; ++to) {
        const int o = o0 + 16 * to + (lane & 15);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = i0 + 16 * ti + 4 * (lane >> 4) + j;
          if (i < Ci && o < Co)
            store_pair<DT>(a.dw, 2 * (((size_t)mode * Ci + i) * Co + o), sc * accr[m][ti][to][j],
                           sc * acci[m][ti][to][j]);
        }
      }
  }
}

// tile shape: the large one when it gives at least 256 workgroups
static bool gradw_small_tiles(const GradWArgs &a) {
  const long big = (long)((a.K + 15) / 16) * ((a.Ci + 31) / 32) * ((a.Co + 31) / 32);
  return big < 256;
}

// hx: the spectra arrive as the half exchange (fp16 / bf16 plans only)
template <int MB, int CT>
static const void *gradw_kernel_t(int dtype, bool hx) {
  switch (dtype) {
    case DT_F32: return hx ? nullptr : (const void *)fno_grad_w<DT_F32, MB, CT, false>;
    case DT_F16: return hx ? (const void *)fno_grad_w<DT_F16, MB, CT, true> : (const void *)fno_grad_w<DT_F16, MB, CT, false>;
    case DT_BF16:
      return hx ? (const void *)fno_grad_w<DT_BF16, MB, CT, true> : (const void *)fno_grad_w<DT_BF16, MB, CT, false>;
  }
  return nullptr;
}

bool gradw_supported(int K) { return (K & 1) == 0; }

hipError_t launch_grad_w(const GradWArgs &a, int dtype, hipStream_t s) {
  FNO_BOUNDS(check_grad_w(a, dtype);)
  const bool small = gradw_small_tiles(a);
  const int MB = small ? 8 : 16, CT = small ? 16 : 32;
  const bool hx = a.xs16 != nullptr;
  const void *k = small ? gradw_kernel_t<8, 16>(dtype, hx) : gradw_kernel_t<16, 32>(dtype, hx);
  if (!k || !gradw_supported(a.K) || (hx && (a.K & 3))) return hipErrorInvalidValue;
  const long gy = (long)((a.Ci + CT - 1) / CT) * ((a.Co + CT - 1) / CT);
  if (gy > 65535) return hipErrorInvalidValue;
  dim3 grid((a.K + MB - 1) / MB, (unsigned)gy);
  void *args[] = {(void *)&a};
  return hipLaunchKernel(k, grid, dim3(kGwT), args, 0, s);
}

}  // namespace fno
