// Device code shared by the FFT kernels of this library (generic-length
// kernels in fft_generic.hpp, fixed-length kernels in fft_fixed.hpp): the radix
// butterflies, twiddle application and memory helpers.
#pragma once

#include "common.hpp"
#include "internal.hpp"

namespace fftmv {
namespace {

// ---------------------------------------------------------------- DFTs
// y_q = sum_p x_p exp(S 2 pi i p q / R), in place, S = -1 forward, +1 inverse.
template <int S, typename T>
__device__ __forceinline__ void dft2(cx<T> &a, cx<T> &b) {
  cx<T> t = a - b;
  a = a + b;
  b = t;
}

template <int S, typename T>
__device__ __forceinline__ void dft3(cx<T> *x) {
  // y_{1,2} = x0 - (x1 + x2)/2 +- S i sin(2 pi / 3) (x1 - x2)
  const T h = T(0.86602540378443864676372317075293618347);  // sqrt(3)/2
  cx<T> t = x[1] + x[2];
  cx<T> m = mk(x[0].re - T(0.5) * t.re, x[0].im - T(0.5) * t.im);
  cx<T> d = x[1] - x[2];
  d = mul_si<S>(mk(h * d.re, h * d.im));
  x[0] = x[0] + t;
  x[1] = m + d;
  x[2] = m - d;
}

template <int S, typename T>
__device__ __forceinline__ void dft4(cx<T> &x0, cx<T> &x1, cx<T> &x2, cx<T> &x3) {
  cx<T> t0 = x0 + x2, t1 = x0 - x2, t2 = x1 + x3, t3 = mul_si<S>(x1 - x3);
  x0 = t0 + t2;
  x2 = t0 - t2;
  x1 = t1 + t3;
  x3 = t1 - t3;
}

template <int S, typename T>
__device__ __forceinline__ void dft8(cx<T> *x) {
  // two length-4 transforms of the even and odd samples, then the
  // exp(S 2 pi i q / 8) twiddles and one radix-2 step
  const T h = T(0.70710678118654752440084436210484903928);  // 1/sqrt(2)
  dft4<S>(x[0], x[2], x[4], x[6]);
  dft4<S>(x[1], x[3], x[5], x[7]);
  cx<T> b1 = x[3], b2 = x[5], b3 = x[7];
  // positions: even transform a_q at x[0],x[2],x[4],x[6]; odd b_q at x[1],x[3],x[5],x[7]
  cx<T> a0 = x[0], a1 = x[2], a2 = x[4], a3 = x[6], b0 = x[1];
  b1 = mk((b1.re - S * b1.im) * h, (b1.im + S * b1.re) * h);   // * (1 + S i)/sqrt 2
  b2 = mul_si<S>(b2);                                          // * S i
  b3 = mk((-b3.re - S * b3.im) * h, (S * b3.re - b3.im) * h);  // * (-1 + S i)/sqrt 2
  x[0] = a0 + b0;
  x[4] = a0 - b0;
  x[1] = a1 + b1;
  x[5] = a1 - b1;
  x[2] = a2 + b2;
  x[6] = a2 - b2;
  x[3] = a3 + b3;
  x[7] = a3 - b3;
}

template <int S, typename T>
__device__ __forceinline__ void dft5(cx<T> *x) {
  // cos and sin of 2 pi / 5 and 4 pi / 5
  const T c1 = T(0.30901699437494742410229341718281905886);
  const T c2 = T(-0.80901699437494742410229341718281905886);
  const T s1 = T(0.95105651629515357211643933337938214340);
  const T s2 = T(0.58778525229247312916870595463907276860);
  cx<T> t1 = x[1] + x[4], t2 = x[2] + x[3], t3 = x[1] - x[4], t4 = x[2] - x[3];
  cx<T> a1 = mk(x[0].re + c1 * t1.re + c2 * t2.re, x[0].im + c1 * t1.im + c2 * t2.im);
  cx<T> a2 = mk(x[0].re + c2 * t1.re + c1 * t2.re, x[0].im + c2 * t1.im + c1 * t2.im);
  cx<T> b1 = mk(s1 * t3.re + s2 * t4.re, s1 * t3.im + s2 * t4.im);
  cx<T> b2 = mk(s2 * t3.re - s1 * t4.re, s2 * t3.im - s1 * t4.im);
  x[0] = x[0] + t1 + t2;
  b1 = mul_si<S>(b1);
  b2 = mul_si<S>(b2);
  x[1] = a1 + b1;
  x[4] = a1 - b1;
  x[2] = a2 + b2;
  x[3] = a2 - b2;
}

template <int S, typename T>
__device__ __forceinline__ void dft7(cx<T> *x) {
  // pairs (p, 7 - p): y_q = a_q + S i b_q and y_{7-q} = a_q - S i b_q with
  // a_q = x0 + sum_p (x_p + x_{7-p}) cos(2 pi p q / 7),
  // b_q = sum_p (x_p - x_{7-p}) sin(2 pi p q / 7), p, q = 1..3
  const T c1 = T(0.62348980185873353052500488400423981063);   // cos(2 pi / 7)
  const T c2 = T(-0.22252093395631440428890256449679475947);  // cos(4 pi / 7)
  const T c3 = T(-0.90096886790241912623610231950744505117);  // cos(6 pi / 7)
  const T s1 = T(0.78183148246802980870844452667405775023);   // sin(2 pi / 7)
  const T s2 = T(0.97492791218182360701813168299393121723);   // sin(4 pi / 7)
  const T s3 = T(0.43388373911755812047576833284835875461);   // sin(6 pi / 7)
  const cx<T> t1 = x[1] + x[6], t2 = x[2] + x[5], t3 = x[3] + x[4];
  const cx<T> u1 = x[1] - x[6], u2 = x[2] - x[5], u3 = x[3] - x[4];
  auto lin = [](T a, cx<T> p, T b, cx<T> q, T c, cx<T> r) {
    return mk(a * p.re + b * q.re + c * r.re, a * p.im + b * q.im + c * r.im);
  };
  const cx<T> a1 = x[0] + lin(c1, t1, c2, t2, c3, t3);
  const cx<T> a2 = x[0] + lin(c2, t1, c3, t2, c1, t3);
  const cx<T> a3 = x[0] + lin(c3, t1, c1, t2, c2, t3);
  const cx<T> b1 = mul_si<S>(lin(s1, u1, s2, u2, s3, u3));
  const cx<T> b2 = mul_si<S>(lin(s2, u1, -s3, u2, -s1, u3));
  const cx<T> b3 = mul_si<S>(lin(s3, u1, -s1, u2, s2, u3));
  x[0] = x[0] + t1 + t2 + t3;
  x[1] = a1 + b1;
  x[6] = a1 - b1;
  x[2] = a2 + b2;
  x[5] = a2 - b2;
  x[3] = a3 + b3;
  x[4] = a3 - b3;
}

template <int R, int S, typename T>
__device__ __forceinline__ void dft(cx<T> *x) {
  if constexpr (R == 2) dft2<S>(x[0], x[1]);
  else if constexpr (R == 3) dft3<S>(x);
  else if constexpr (R == 4) dft4<S>(x[0], x[1], x[2], x[3]);
  else if constexpr (R == 5) dft5<S>(x);
  else if constexpr (R == 7) dft7<S>(x);
  else dft8<S>(x);
}

template <typename T, int R, int S>
__device__ __forceinline__ void twiddle(cx<T> *v, int k, int twstep, const cx<T> *__restrict__ tw) {
#pragma unroll
  for (int q = 1; q < R; ++q) {
    cx<T> w = tw[k * q * twstep];
    v[q] = S < 0 ? cmul(v[q], w) : cmulc(v[q], w);
  }
}

// Element at base + index. OFF32: the index fits 32 bits in bytes, so the
// address is a uniform base plus one 32-bit per-lane offset (one VGPR per
// load in flight instead of a 64-bit address pair).
template <bool OFF32, typename E>
__device__ __forceinline__ E load_elem(const E *base, int64_t index) {
  if constexpr (OFF32)
    return *reinterpret_cast<const E *>(reinterpret_cast<const char *>(base) +
                                        static_cast<uint32_t>(index) * static_cast<uint32_t>(sizeof(E)));
  else
    return base[index];
}
template <bool OFF32, typename E>
__device__ __forceinline__ void store_elem(E *base, int64_t index, E v) {
  if constexpr (OFF32)
    *reinterpret_cast<E *>(reinterpret_cast<char *>(base) +
                           static_cast<uint32_t>(index) * static_cast<uint32_t>(sizeof(E))) = v;
  else
    base[index] = v;
}

__device__ __forceinline__ void store_stream(cx<float> *p, cx<float> v) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  __builtin_nontemporal_store(f32x2{v.re, v.im}, reinterpret_cast<f32x2 *>(p));
}
__device__ __forceinline__ void store_stream2(cx<float> *p, cx<float> v0, cx<float> v1) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(f32x4{v0.re, v0.im, v1.re, v1.im}, reinterpret_cast<f32x4 *>(p));
}
__device__ __forceinline__ void store_stream(cx<double> *p, cx<double> v) {
  typedef double f64x2 __attribute__((ext_vector_type(2)));
  __builtin_nontemporal_store(f64x2{v.re, v.im}, reinterpret_cast<f64x2 *>(p));
}

// byte extent below 4 GiB: 32-bit offsets are exact
inline bool fits_32bit(int64_t rows, int64_t ld, int64_t esz) { return rows * ld * esz < (int64_t(1) << 32); }

}  // namespace
}  // namespace fftmv
