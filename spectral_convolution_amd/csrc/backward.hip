// backward.hip - the kernels of the layer's backward pass that the forward
// path does not already provide.
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
// fno_conj_transpose forms W^H (only where the adjoint contraction cannot
// read W itself); fno_grad_w is the per-mode batch reduction on complex fp32
// spectra, fno_grad_w_hx the same on the half exchange (fp16 matrix cores).

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

template <int DT, int MB, int CT>
__global__ __launch_bounds__(kGwT) __attribute__((amdgpu_waves_per_eu(2))) void fno_grad_w(GradWArgs a) {
  using G = GwShape<MB, CT>;
  constexpr int MW = G::MW, NT = G::NT;
  __shared__ float2 xs[MB * G::S], gs[MB * G::S];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int K = a.K, Ci = a.Ci, Co = a.Co, B = a.B;
  // workgroups of one mode block are gridDim.x apart: with gridDim.x a
  // multiple of 8 they share an XCD (and its L2), where the second read of
  // each spectra row hits (measured 4 % faster than also keeping the mode
  // blocks of one 128-byte line on one XCD)
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

  gw_u32x4 px[G::U], pg[G::U];
  auto fetch = [&](int st) {
    gw_fetch<MB, CT>(a.xs, Ci, K, B, st, k0, i0, tid, px);
    gw_fetch<MB, CT>(a.gs, Co, K, B, st, k0, o0, tid, pg);
  };
  fetch(0);
  for (int st = 0; st < nst; ++st) {
    gw_put<MB, CT>(xs, tid, px);
    gw_put<MB, CT>(gs, tid, pg);
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

// ------------------------------------------ dw on fp16 matrix cores
//
// For the half exchange (fp16 / bf16 plans; the exchanged spectra are fp16
// pairs either way, the gradient is rounded to the plan's dtype): the same per-mode product with the
// batch as the reduction, on v_mfma_f32_16x16x32_f16. In real form, per mode,
// M = i and K = (b, re/im); two products share the A operand
//   A[i][(b,0)] = Re X,  A[i][(b,1)] = Im X,
//   B0[(b,0)][o] = Re G, B0[(b,1)][o] = Im G   giving Re sum_b conj(X) G,
//   B1[(b,0)][o] = Im G, B1[(b,1)][o] = -Re G  giving Im sum_b conj(X) G;
// a B1 fragment is the B0 fragment with the halves of every pair swapped and
// the new high half negated, so each lane ends with (re, im) of its outputs.
// The exchanged spectra are fp16 pairs scaled per plane by 2^e; every input
// channel row i is brought to the smallest exponent over the batch, EX_i (its
// largest plane keeps its scale, the others are multiplied by 2^-d, d >= 0:
// one correctly rounded fp16 product, the same value as the decode to fp32
// and back), and likewise every output channel row o to EG_o, so one product
// sums the whole batch in one scale, undone per (i, o) at the end. A
// workgroup (4 waves) owns 8 modes x 32 input x 32 output channels and
// streams the batch in stages of 16 rows (one 32-deep K block): 16-byte loads
// of 4 modes' pairs one stage ahead, staged into LDS as fragment rows of 48
// halves (32 + 16 pad: a fragment read is conflict-free with the row pitch
// 2 mod 4 16-byte units); wave w multiplies modes 2 w and 2 w + 1.
constexpr int kGhM = 8;        // modes per workgroup
constexpr int kGhC = 32;       // input and output channels per workgroup
constexpr int kGhB = 16;       // batch rows per stage
constexpr int kGhP = 48;       // halves per staged fragment row
constexpr int kGhS = 32 * kGhP + 8;   // halves per staged mode (rows + pad)
constexpr int kGhU = kGhB * kGhC * kGhM / 4 / kGwT;  // 16-byte units per thread and operand (4)

typedef _Float16 gh_f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 gh_f16x2 __attribute__((ext_vector_type(2)));

// Units of a thread (lane l, wave w): mode quad q = l % 2, batch row
// bl = (l / 2) % 16 of the stage and channels cb + 8 v, v < 4, with
// cb = 4 (w / 2) + w % 2 + 2 (l / 32). A 4-byte LDS store serves 32 lanes per
// pass over 32 banks; for lanes 0..31 (and 32..63) the words of one store are
// the 16 batch rows on consecutive banks and, for the other mode quad, 4
// staged modes on (3088 words, 16 banks mod 32).
struct GhLane {
  int q, bl, cb;
};

__device__ __forceinline__ GhLane gh_lane(int tid) {
  const int lane = tid & 63, wv = tid >> 6;
  return GhLane{lane & 1, (lane >> 1) & 15, 4 * (wv >> 1) + (wv & 1) + 2 * (lane >> 5)};
}

// one stage of one operand (nc channels, tile origin c0)
__device__ __forceinline__ void gh_fetch(const uint32_t *src, const int *ex, int nc, int K, int B, int st, int k0,
                                         int c0, const GhLane &g, gw_u32x4 (&p)[kGhU], int (&e)[kGhU]) {
  const int b = st * kGhB + g.bl, mode = k0 + 4 * g.q;
  const uint32_t *sb = src + (size_t)st * kGhB * nc * K;  // first plane row of the stage
  const int *eb = ex + (size_t)st * kGhB * nc;
  const int row = g.bl * nc + c0 + g.cb;                   // plane row within the stage, v = 0
#pragma unroll
  for (int v = 0; v < kGhU; ++v) {
    const bool ok = b < B && c0 + g.cb + 8 * v < nc && mode < K;
    const gw_u32x4 t = *reinterpret_cast<const gw_u32x4 *>(sb + (ok ? (row + 8 * v) * K + mode : 0));
    p[v] = ok ? t : gw_u32x4{0u, 0u, 0u, 0u};
    e[v] = eb[ok ? row + 8 * v : 0];
  }
}

// bring one stage to the common exponents em[v] of the thread's channels and
// store it as fragment rows st_[mode][c][2 b + re/im]
__device__ __forceinline__ void gh_put(uint16_t *st_, const GhLane &g, const int (&em)[kGhU],
                                       const gw_u32x4 (&p)[kGhU], const int (&e)[kGhU]) {
  uint32_t *w = reinterpret_cast<uint32_t *>(st_ + 4 * g.q * kGhS + g.cb * kGhP) + g.bl;
#pragma unroll
  for (int v = 0; v < kGhU; ++v) {
    const int d = max(0, e[v] - em[v]);  // invalid units hold zeros
    // 2^-d in fp16: normal for d <= 14, subnormal up to d = 24
    const uint32_t sbits = d <= 14 ? (15u - d) << 10 : (d <= 24 ? 1u << (24 - d) : 0u);
    const gh_f16x2 s = __builtin_bit_cast(gh_f16x2, sbits | (sbits << 16));
    // the words as scalars: a bit cast of a vector element read element 0
    const uint32_t pw[4] = {p[v].x, p[v].y, p[v].z, p[v].w};
    uint32_t r[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) r[t] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(gh_f16x2, pw[t]) * s);
    if (d > 24) {
      // beyond one fp16 factor: through fp32
      const float f = pow2f(-d);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const gh_f16x2 h = __builtin_bit_cast(gh_f16x2, pw[t]);
        const gh_f16x2 o = {(_Float16)((float)h.x * f), (_Float16)((float)h.y * f)};
        r[t] = __builtin_bit_cast(uint32_t, o);
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) w[t * (kGhS / 2) + v * 8 * (kGhP / 2)] = r[t];
  }
}

template <int DT>
__global__ __launch_bounds__(kGwT) __attribute__((amdgpu_waves_per_eu(3))) void fno_grad_w_hx(GradWArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[kGhM * kGhS], gs[kGhM * kGhS];
  __shared__ int exm[kGhC], egm[kGhC];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int K = a.K, Ci = a.Ci, Co = a.Co, B = a.B;
  // workgroup h runs on XCD h % 8; with the count a multiple of 8, XCD x
  // takes the x-th eighth of the blocks in order (tiles of a mode block
  // fastest), so the four mode blocks that share a 128-byte spectra line and
  // the tiles that re-read it all go through one L2
  const int nto = (Co + kGhC - 1) / kGhC, nti = (Ci + kGhC - 1) / kGhC;
  const int ng = gridDim.x, h = blockIdx.x;
  const int L = (ng & 7) == 0 ? (h & 7) * (ng >> 3) + (h >> 3) : h;
  const int tile = L % (nti * nto);
  const int k0 = (L / (nti * nto)) * kGhM;
  const int i0 = (tile / nto) * kGhC, o0 = (tile % nto) * kGhC;
  const int nst = (B + kGhB - 1) / kGhB;
  const GhLane g = gh_lane(tid);

  gw_u32x4 px[kGhU], pg[kGhU];
  int ex[kGhU], eg[kGhU];
  gh_fetch(a.xs16, a.xexp, Ci, K, B, 0, k0, i0, g, px, ex);
  gh_fetch(a.gs16, a.gexp, Co, K, B, 0, k0, o0, g, pg, eg);
  // common exponent of every channel row over the batch: four threads per
  // row, rows 0..31 the input channels, 32..63 the output channels
  {
    const int row = tid >> 2, part = tid & 3;
    const bool isx = row < kGhC;
    const int c = (isx ? i0 : o0) + (row & (kGhC - 1)), nc = isx ? Ci : Co;
    const int *exs = isx ? a.xexp : a.gexp;
    int m = 1 << 20;
    if (c < nc) {
#pragma unroll 8
      for (int b = part; b < B; b += 4) m = min(m, exs[(size_t)b * nc + c]);
    }
    m = min(m, __shfl_xor(m, 1, 64));
    m = min(m, __shfl_xor(m, 2, 64));
    if (part == 0) (isx ? exm : egm)[row & (kGhC - 1)] = m < (1 << 20) ? m : 0;
  }
  __syncthreads();
  int emx[kGhU], emg[kGhU];
#pragma unroll
  for (int v = 0; v < kGhU; ++v) {
    emx[v] = exm[g.cb + 8 * v];
    emg[v] = egm[g.cb + 8 * v];
  }

  v4f acc[2][2][2][2];  // [mode of the wave][i tile][o tile][re, im]
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int ot = 0; ot < 2; ++ot) acc[m][mt][ot][0] = acc[m][mt][ot][1] = v4f{0.f, 0.f, 0.f, 0.f};

  // fragment of lane l: row 16 t + l % 16, halves 8 (l / 16) .. + 7
  const int fr = (lane & 15) * kGhP + 8 * (lane >> 4);
  for (int st = 0; st < nst; ++st) {
    gh_put(xs, g, emx, px, ex);
    gh_put(gs, g, emg, pg, eg);
    if (st + 1 < nst) {
      gh_fetch(a.xs16, a.xexp, Ci, K, B, st + 1, k0, i0, g, px, ex);
      gh_fetch(a.gs16, a.gexp, Co, K, B, st + 1, k0, o0, g, pg, eg);
    }
    __syncthreads();
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      const int m = 2 * wv + mm;
      gw_u32x4 af[2], b0[2], b1[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        af[t] = *reinterpret_cast<const gw_u32x4 *>(xs + m * kGhS + 16 * t * kGhP + fr);
        b0[t] = *reinterpret_cast<const gw_u32x4 *>(gs + m * kGhS + 16 * t * kGhP + fr);
#pragma unroll
        for (int j = 0; j < 4; ++j) b1[t][j] = __builtin_amdgcn_alignbit(b0[t][j], b0[t][j], 16) ^ 0x80000000u;
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int ot = 0; ot < 2; ++ot) {
          const gh_f16x8 av = __builtin_bit_cast(gh_f16x8, af[mt]);
          acc[mm][mt][ot][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(gh_f16x8, b0[ot]),
                                                                      acc[mm][mt][ot][0], 0, 0, 0);
          acc[mm][mt][ot][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(gh_f16x8, b1[ot]),
                                                                      acc[mm][mt][ot][1], 0, 0, 0);
        }
    }
    __syncthreads();
  }

  // accumulator register j of lane l: i = 16 mt + 4 (l / 16) + j,
  // o = 16 ot + l % 16; 16 lanes store 16 consecutive outputs
  float fx[2][4], fg[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    fg[t] = pow2f(-egm[16 * t + (lane & 15)]);
#pragma unroll
    for (int j = 0; j < 4; ++j) fx[t][j] = pow2f(-exm[16 * t + 4 * (lane >> 4) + j]);
  }
#pragma unroll
  for (int mm = 0; mm < 2; ++mm) {
    const int mode = k0 + 2 * wv + mm;
    const float sc = a.scale * ((mode % a.mlast) == 0 ? 1.0f : 2.0f);
#pragma unroll
    for (int ot = 0; ot < 2; ++ot) {
      const int o = o0 + 16 * ot + (lane & 15);
      const float fo = sc * fg[ot];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = i0 + 16 * mt + 4 * (lane >> 4) + j;
          if (mode < K && i < Ci && o < Co) {
            const float f = fo * fx[mt][j];
            store_pair<DT>(a.dw, 2 * (((size_t)mode * Ci + i) * Co + o), acc[mm][mt][ot][0][j] * f,
                           acc[mm][mt][ot][1][j] * f);
          }
        }
    }
  }
}

// tile shape: the large one when it gives at least 256 workgroups
static bool gradw_small_tiles(const GradWArgs &a) {
  const long big = (long)((a.K + 15) / 16) * ((a.Ci + 31) / 32) * ((a.Co + 31) / 32);
  return big < 256;
}

template <int MB, int CT>
static const void *gradw_kernel_t(int dtype) {
  switch (dtype) {
    case DT_F32: return (const void *)fno_grad_w<DT_F32, MB, CT>;
    case DT_F16: return (const void *)fno_grad_w<DT_F16, MB, CT>;
    case DT_BF16: return (const void *)fno_grad_w<DT_BF16, MB, CT>;
  }
  return nullptr;
}

bool gradw_supported(int K) { return (K & 1) == 0; }

// the half-exchange weight gradient: fp16 / bf16 plans, 16-byte mode quads, and the
// per-stage element offsets (16 batch rows of a spectra operand) in int
bool gradw_hx_supported(int dtype, int K, int Ci, int Co) {
  return (dtype == DT_F16 || dtype == DT_BF16) && K % 4 == 0 && (long)kGhB * (Ci > Co ? Ci : Co) * K < 0x7fffffffL;
}

hipError_t launch_grad_w(const GradWArgs &a, int dtype, hipStream_t s) {
  FNO_BOUNDS(check_grad_w(a, dtype);)
  if (a.xs16) {
    // half exchange: the fp16 matrix-core kernel
    const long n = (long)((a.K + kGhM - 1) / kGhM) * ((a.Ci + kGhC - 1) / kGhC) * ((a.Co + kGhC - 1) / kGhC);
    if (!gradw_hx_supported(dtype, a.K, a.Ci, a.Co) || n > 0x7fffffffL) return hipErrorInvalidValue;
    void *args[] = {(void *)&a};
    const void *k = dtype == DT_F16 ? (const void *)fno_grad_w_hx<DT_F16> : (const void *)fno_grad_w_hx<DT_BF16>;
    return hipLaunchKernel(k, dim3((unsigned)n), dim3(kGwT), args, 0, s);
  }
  const bool small = gradw_small_tiles(a);
  const int MB = small ? 8 : 16, CT = small ? 16 : 32;
  const void *k = small ? gradw_kernel_t<8, 16>(dtype) : gradw_kernel_t<16, 32>(dtype);
  if (!k || !gradw_supported(a.K)) return hipErrorInvalidValue;
  const long gy = (long)((a.Ci + CT - 1) / CT) * ((a.Co + CT - 1) / CT);
  if (gy > 65535) return hipErrorInvalidValue;
  dim3 grid((a.K + MB - 1) / MB, (unsigned)gy);
  void *args[] = {(void *)&a};
  return hipLaunchKernel(k, grid, dim3(kGwT), args, 0, s);
}

}  // namespace fno
