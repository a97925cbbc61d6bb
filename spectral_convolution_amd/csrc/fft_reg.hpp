// fft_reg.hpp - complex FFTs held entirely in one thread's registers.
//
// The building block of the pruned transforms: a length-MP (power of two,
// MP <= 32) DFT computed by radix-4 decimation-in-frequency stages (a final
// radix-2 stage when log2(MP) is odd), fully unrolled so that every twiddle
// is a compile-time constant and multiplications by 1, -1, +-i are dropped.
// The output is in bit-reversed order: X[k] = a[bitrev(k)].
//
// Twiddles are computed at compile time in double precision from the
// definition (Taylor series on an octant-reduced angle) and rounded to fp32.
// Forward transforms use exp(-2 pi i k n / N), inverse ones exp(+2 pi i k n /
// N) without the 1/N factor.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

namespace fno {

// ------------------------------------------------------------ compile-time trig

constexpr double kPi = 3.14159265358979323846264338327950288;

// sin and cos of |x| <= pi/4 by Taylor series (converged to double precision)
constexpr double ce_sin_small(double x) {
  double term = x, sum = x;
  for (int n = 1; n < 14; ++n) {
    term *= -x * x / ((2.0 * n) * (2.0 * n + 1.0));
    sum += term;
  }
  return sum;
}
constexpr double ce_cos_small(double x) {
  double term = 1.0, sum = 1.0;
  for (int n = 1; n < 14; ++n) {
    term *= -x * x / ((2.0 * n - 1.0) * (2.0 * n));
    sum += term;
  }
  return sum;
}

struct ce_cs {
  double c, s;
};

// cos and sin of 2*pi*k/n, exact quadrant reduction in integers
constexpr ce_cs ce_cossin_2pi(long k, long n) {
  long r = ((k % n) + n) % n;
  long q = (4 * r) / n;        // quadrant 0..3
  long rem = 4 * r - q * n;    // angle within quadrant = (pi/2) * rem / n
  double ca = 0, sa = 0;
  if (2 * rem <= n) {
    double a = (kPi / 2.0) * (double)rem / (double)n;
    ca = ce_cos_small(a);
    sa = ce_sin_small(a);
  } else {
    double b = (kPi / 2.0) * (double)(n - rem) / (double)n;
    ca = ce_sin_small(b);
    sa = ce_cos_small(b);
  }
  if (q == 0) return {ca, sa};
  if (q == 1) return {-sa, ca};
  if (q == 2) return {-ca, -sa};
  return {sa, -ca};
}

// ------------------------------------------------------------- complex helpers

__device__ __forceinline__ float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ float2 csub(float2 a, float2 b) { return make_float2(a.x - b.x, a.y - b.y); }
__device__ __forceinline__ float2 cconj(float2 a) { return make_float2(a.x, -a.y); }
__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
  return make_float2(fmaf(a.x, b.x, -a.y * b.y), fmaf(a.x, b.y, a.y * b.x));
}
// a * conj(b)
__device__ __forceinline__ float2 cmulc(float2 a, float2 b) {
  return make_float2(fmaf(a.x, b.x, a.y * b.y), fmaf(a.y, b.x, -a.x * b.y));
}
// acc * w + d
__device__ __forceinline__ float2 cfma(float2 acc, float2 w, float2 d) {
  return make_float2(fmaf(acc.x, w.x, fmaf(-acc.y, w.y, d.x)),
                     fmaf(acc.x, w.y, fmaf(acc.y, w.x, d.y)));
}

// multiply by -i (forward) or +i (inverse)
template <bool INV>
__device__ __forceinline__ float2 mul_mi(float2 a) {
  if constexpr (INV) return make_float2(-a.y, a.x);
  else return make_float2(a.y, -a.x);
}

// a * w where w = exp(-+2 pi i K / N), specialised at compile time
template <int K, int N, bool INV>
__device__ __forceinline__ float2 twmul(float2 a) {
  constexpr int k = ((K % N) + N) % N;
  if constexpr (k == 0) {
    return a;
  } else if constexpr (2 * k == N) {
    return make_float2(-a.x, -a.y);
  } else if constexpr (4 * k == N) {
    return mul_mi<INV>(a);
  } else if constexpr (4 * k == 3 * N) {
    return mul_mi<!INV>(a);
  } else {
    constexpr ce_cs cs = ce_cossin_2pi(k, N);
    constexpr float c = (float)cs.c;
    constexpr float s = INV ? (float)cs.s : (float)(-cs.s);  // w = c + i s
    if constexpr (8 * k == N || 8 * k == 3 * N || 8 * k == 5 * N || 8 * k == 7 * N) {
      // |c| == |s| == 1/sqrt(2): two adds and two multiplies
      constexpr float h = c > 0 ? c : -c;
      constexpr float sc = c > 0 ? 1.0f : -1.0f;
      constexpr float ss = s > 0 ? 1.0f : -1.0f;
      // re = c a.x - s a.y, im = s a.x + c a.y
      float re = sc * a.x - ss * a.y;
      float im = ss * a.x + sc * a.y;
      return make_float2(h * re, h * im);
    } else {
      return make_float2(fmaf(a.x, c, -a.y * s), fmaf(a.x, s, a.y * c));
    }
  }
}

// --------------------------------------------------------- static loop helper

template <int I>
using ic = std::integral_constant<int, I>;

template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (B < E) {
    f(ic<B>{});
    static_for<B + 1, E>(f);
  }
}

constexpr int ilog2(int n) { return n <= 1 ? 0 : 1 + ilog2(n / 2); }

constexpr int bitrev(int k, int bits) {
  int r = 0;
  for (int i = 0; i < bits; ++i) {
    r = (r << 1) | (k & 1);
    k >>= 1;
  }
  return r;
}

// ------------------------------------------------------------------ DIF stages

template <int N, int L, bool INV>
__device__ __forceinline__ void dif_stages(float2 (&a)[N]) {
  if constexpr (L >= 4) {
    constexpr int Q = L / 4;
    static_for<0, N / L>([&](auto blk) {
      static_for<0, Q>([&](auto jj) {
        constexpr int j = decltype(jj)::value;
        constexpr int b = decltype(blk)::value * L + j;
        float2 a0 = a[b], a1 = a[b + Q], a2 = a[b + 2 * Q], a3 = a[b + 3 * Q];
        float2 t0 = cadd(a0, a2), t1 = csub(a0, a2);
        float2 t2 = cadd(a1, a3), t3 = mul_mi<INV>(csub(a1, a3));
        a[b] = cadd(t0, t2);
        a[b + Q] = twmul<2 * j, L, INV>(csub(t0, t2));
        a[b + 2 * Q] = twmul<j, L, INV>(cadd(t1, t3));
        a[b + 3 * Q] = twmul<3 * j, L, INV>(csub(t1, t3));
      });
    });
    dif_stages<N, L / 4, INV>(a);
  } else if constexpr (L == 2) {
    static_for<0, N / 2>([&](auto blk) {
      constexpr int b = 2 * decltype(blk)::value;
      float2 u = a[b], v = a[b + 1];
      a[b] = cadd(u, v);
      a[b + 1] = csub(u, v);
    });
  }
}

// In-place length-N DFT of a[] (natural order in, bit-reversed order out).
template <int N, bool INV>
__device__ __forceinline__ void fft_reg(float2 (&a)[N]) {
  static_assert((N & (N - 1)) == 0 && N >= 1 && N <= 64, "N must be a power of two <= 64");
  dif_stages<N, N, INV>(a);
}

}  // namespace fno
