// Device-side helpers shared by the fftmv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fftmv {

constexpr int kWave = 64;
constexpr int kBlock = 256;  // the default workgroup size
constexpr int kXcds = 8;     // MI355X: 8 accelerator complex dies, one L2 each

template <typename T>
struct alignas(2 * sizeof(T)) cx {
  T re, im;
};

template <typename T>
__device__ __forceinline__ cx<T> mk(T re, T im) {
  cx<T> r;
  r.re = re;
  r.im = im;
  return r;
}
template <typename T>
__device__ __forceinline__ cx<T> operator+(cx<T> a, cx<T> b) {
  return mk(a.re + b.re, a.im + b.im);
}
template <typename T>
__device__ __forceinline__ cx<T> operator-(cx<T> a, cx<T> b) {
  return mk(a.re - b.re, a.im - b.im);
}
template <typename T>
__device__ __forceinline__ cx<T> cmul(cx<T> a, cx<T> b) {
  return mk(a.re * b.re - a.im * b.im, a.re * b.im + a.im * b.re);
}
// a * conj(b)
template <typename T>
__device__ __forceinline__ cx<T> cmulc(cx<T> a, cx<T> b) {
  return mk(a.re * b.re + a.im * b.im, a.im * b.re - a.re * b.im);
}
template <typename T>
__device__ __forceinline__ cx<T> conj(cx<T> a) {
  return mk(a.re, -a.im);
}
template <typename T>
__device__ __forceinline__ cx<T> scale(cx<T> a, T s) {
  return mk(a.re * s, a.im * s);
}
// multiply by s*i, s = +1 or -1
template <int S, typename T>
__device__ __forceinline__ cx<T> mul_si(cx<T> a) {
  return S > 0 ? mk(-a.im, a.re) : mk(a.im, -a.re);
}
template <typename D, typename S>
__device__ __forceinline__ cx<D> cvt(cx<S> a) {
  return mk(static_cast<D>(a.re), static_cast<D>(a.im));
}

// Value of a double after rounding to binary32 and back (RN-even), used
// where a stage boundary has an FP32 stage on one side.
__device__ __forceinline__ double round_f32(double x) { return static_cast<double>(static_cast<float>(x)); }

// ---------------------------------------------------------------- DPP
// Cross-lane moves inside one row of 16 lanes (gfx9 DPP controls).
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm(1,0,3,2)
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm(2,3,0,1)
constexpr int kDppRowHalfMirror = 0x141; // lane i <-> 7-i within each 8
constexpr int kDppRowMirror = 0x140;     // lane i <-> 15-i within each 16

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
struct u32x2 {
  int x, y;
};

template <int CTRL>
__device__ __forceinline__ double dpp(double x) {
  u32x2 v = __builtin_bit_cast(u32x2, x);
  v.x = __builtin_amdgcn_update_dpp(0, v.x, CTRL, 0xF, 0xF, false);
  v.y = __builtin_amdgcn_update_dpp(0, v.y, CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, v);
}
__device__ __forceinline__ float readlane(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}
__device__ __forceinline__ double readlane(double x, int l) {
  u32x2 v = __builtin_bit_cast(u32x2, x);
  v.x = __builtin_amdgcn_readlane(v.x, l);
  v.y = __builtin_amdgcn_readlane(v.y, l);
  return __builtin_bit_cast(double, v);
}

// Sum over the 64 lanes of a wave, returned (uniform) to every lane. Four
// DPP butterfly steps give every lane its 16-lane row sum; the four row sums
// are then added in a fixed order, so the result is bitwise reproducible.
template <typename T>
__device__ __forceinline__ T wave_sum(T x) {
  x = x + dpp<kDppQuadXor1>(x);
  x = x + dpp<kDppQuadXor2>(x);
  x = x + dpp<kDppRowHalfMirror>(x);
  x = x + dpp<kDppRowMirror>(x);
  return (readlane(x, 0) + readlane(x, 16)) + (readlane(x, 32) + readlane(x, 48));
}

// Hardware dispatches workgroup b of a grid to XCD b % 8. Renumber so that
// each XCD receives one contiguous range of logical workgroup ids: work that
// shares an operand (all tasks of one frequency) then shares one L2.
__device__ __forceinline__ int64_t xcd_contiguous_block(int64_t b, int64_t nblocks) {
  int64_t per = nblocks / kXcds, rem = nblocks % kXcds;
  int64_t x = b % kXcds, i = b / kXcds;
  return x < rem ? x * (per + 1) + i : rem * (per + 1) + (x - rem) * per + i;
}

}  // namespace fftmv
