// Stage 3 of "Mixed-precision FFTMatvec performance optimization on AMD
// GPUs", section 1.1: one complex GEMV per frequency against the frequency
// blocks Fhat [K][Nd][ldF] (row-major per frequency, frequency-major
// overall). Section 1.2 asks for both the plain product (F) and the
// conjugate-transpose product on short-wide blocks (F*, Nd << Nm).
//
// Both kernels stream Fhat exactly once with 16-byte loads (two complex64
// or one complex128 per lane) and carry 1 flop per byte (complex64) or 0.5
// (complex128): they are bound by HBM bandwidth, far from the vector-ALU
// and matrix-core limits, so no MFMA is used.
//
// FP32 sums use many short chains (lanes x unrolled slots) and a tree at the
// end, never one long serial chain: with n = 5000 a single FP32 chain alone
// would cost ~1e-6 relative error.
#include "common.hpp"
#include "internal.hpp"

namespace fftmv {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));

template <typename T>
struct Vec16;
template <>
struct Vec16<float> {
  using type = f32x4;  // two complex64
  static constexpr int n = 2;
};
template <>
struct Vec16<double> {
  using type = f64x2;  // one complex128
  static constexpr int n = 1;
};

__device__ __forceinline__ void split(const f32x4 &f, cx<float> *o) {
  o[0] = mk(f.x, f.y);
  o[1] = mk(f.z, f.w);
}
__device__ __forceinline__ void split(const f64x2 &f, cx<double> *o) { o[0] = mk(f.x, f.y); }

// Fhat is read once: non-temporal loads keep it from evicting the reused
// per-frequency vectors from the caches.
__device__ __forceinline__ f32x4 load_stream(const f32x4 *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ f64x2 load_stream(const f64x2 *p) { return __builtin_nontemporal_load(p); }

// The Vec16<T>::n complex entries of the input vector that line up with
// 16-byte vector j of a row, converted to T.
template <typename T, typename In>
__device__ __forceinline__ void load_x(const cx<In> *__restrict__ x, int64_t j, cx<T> *o) {
  if constexpr (sizeof(T) == 4) {
    split(reinterpret_cast<const f32x4 *>(x)[j], o);
  } else if constexpr (sizeof(In) == 8) {
    split(reinterpret_cast<const f64x2 *>(x)[j], o);
  } else {
    o[0] = cvt<double>(x[j]);
  }
}

template <typename T>
__device__ __forceinline__ void store_y(void *y, int64_t idx, bool f32, cx<T> v) {
  if (f32)
    static_cast<cx<float> *>(y)[idx] = cvt<float>(v);
  else
    static_cast<cx<double> *>(y)[idx] = cvt<double>(v);
}

// ------------------------------------------------------------------ F
// v_k[r] = sum_c Fhat_k[r][c] m_k[c].
// One wave per task = (frequency k, R consecutive rows). The wave walks the
// rows side by side: lane l takes 16-byte vectors l, l+64, ... of each row,
// so each load instruction reads 1 KiB contiguous per row, and the matching
// piece of m_k is loaded once for all R rows. U vectors per row are in flight
// per step. Per-lane partial sums are closed with wave_sum (DPP).
template <typename T, typename In, int R, int U>
__global__ __launch_bounds__(kBlock) void sbgemv_n_kernel(const typename Vec16<T>::type *__restrict__ F,
                                                          const cx<In> *__restrict__ x, void *__restrict__ y,
                                                          int64_t Nd, int64_t ldF_vec, int64_t nvec, int64_t ldx,
                                                          int64_t ldy, bool y_f32, int64_t ngroups, int64_t ntasks,
                                                          int64_t nblocks) {
  using V = typename Vec16<T>::type;
  constexpr int NV = Vec16<T>::n;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t task = xcd_contiguous_block(blockIdx.x, nblocks) * (kBlock / kWave) + (threadIdx.x / kWave);
  if (task >= ntasks) return;
  const int64_t k = task / ngroups;
  const int64_t r0 = (task - k * ngroups) * R;

  const V *rows[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    int64_t r = r0 + i < Nd ? r0 + i : Nd - 1;  // tail group: re-read the last row, never store it
    rows[i] = F + (k * Nd + r) * ldF_vec;
  }
  const cx<In> *xk = x + k * ldx;

  cx<T> acc[R][U][NV];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < NV; ++e) acc[i][u][e] = mk(T(0), T(0));

  int64_t j = lane;
  for (; j + (U - 1) * kWave < nvec; j += U * kWave) {
    cx<T> xv[U][NV];
    V fv[U][R];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < R; ++i) fv[u][i] = load_stream(rows[i] + j + u * kWave);
#pragma unroll
    for (int u = 0; u < U; ++u) load_x<T, In>(xk, j + u * kWave, xv[u]);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < R; ++i) {
        cx<T> f[NV];
        split(fv[u][i], f);
#pragma unroll
        for (int e = 0; e < NV; ++e) acc[i][u][e] = acc[i][u][e] + cmul(f[e], xv[u][e]);
      }
  }
  for (; j < nvec; j += kWave) {
    cx<T> xv[NV];
    load_x<T, In>(xk, j, xv);
#pragma unroll
    for (int i = 0; i < R; ++i) {
      cx<T> f[NV];
      split(load_stream(rows[i] + j), f);
#pragma unroll
      for (int e = 0; e < NV; ++e) acc[i][0][e] = acc[i][0][e] + cmul(f[e], xv[e]);
    }
  }

#pragma unroll
  for (int i = 0; i < R; ++i) {
    // pairwise tree over the U*NV chains of this lane
    cx<T> part[U * NV];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < NV; ++e) part[u * NV + e] = acc[i][u][e];
#pragma unroll
    for (int w = 1; w < U * NV; w *= 2)
#pragma unroll
      for (int q = 0; q + w < U * NV; q += 2 * w) part[q] = part[q] + part[q + w];
    cx<T> s = mk(wave_sum(part[0].re), wave_sum(part[0].im));
    if (lane == 0 && r0 + i < Nd) store_y(y, k * ldy + r0 + i, y_f32, s);
  }
}

// ------------------------------------------------------------------ F*
// w_k[c] = sum_r conj(Fhat_k[r][c]) d_k[r].
// One workgroup per (frequency k, 256 consecutive 16-byte column vectors):
// each lane owns one vector (two complex64 columns or one complex128 column)
// and walks down all Nd rows, U rows in flight; no cross-lane reduction.
// d_k[r] is the same for the whole workgroup (a uniform load). Row r feeds
// chain r mod U (the last Nd mod U rows feed chain 0), and the U chains are
// closed with a tree.
template <typename T, typename In, int U>
__global__ __launch_bounds__(kBlock) void sbgemv_c_kernel(const typename Vec16<T>::type *__restrict__ F,
                                                          const cx<In> *__restrict__ x, void *__restrict__ y,
                                                          int64_t Nd, int64_t ldF_vec, int64_t nvec, int64_t ldx,
                                                          int64_t ldy, bool y_f32, int64_t nchunks, int64_t nblocks) {
  using V = typename Vec16<T>::type;
  constexpr int NV = Vec16<T>::n;
  const int64_t blk = xcd_contiguous_block(blockIdx.x, nblocks);
  const int64_t k = blk / nchunks;
  const int64_t j = (blk - k * nchunks) * kBlock + threadIdx.x;
  const bool valid = j < nvec;
  const V *col = F + k * Nd * ldF_vec + (valid ? j : nvec - 1);
  const cx<In> *xk = x + k * ldx;

  cx<T> acc[U][NV];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int e = 0; e < NV; ++e) acc[u][e] = mk(T(0), T(0));

  int64_t r = 0;
  for (; r + U <= Nd; r += U) {
    V fv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) fv[u] = load_stream(col + (r + u) * ldF_vec);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      cx<T> d = cvt<T>(xk[r + u]);
      cx<T> f[NV];
      split(fv[u], f);
#pragma unroll
      for (int e = 0; e < NV; ++e) acc[u][e] = acc[u][e] + cmulc(d, f[e]);
    }
  }
  for (; r < Nd; ++r) {  // fewer than U rows left
    cx<T> d = cvt<T>(xk[r]);
    cx<T> f[NV];
    split(load_stream(col + r * ldF_vec), f);
#pragma unroll
    for (int e = 0; e < NV; ++e) acc[0][e] = acc[0][e] + cmulc(d, f[e]);
  }

#pragma unroll
  for (int w = 1; w < U; w *= 2)
#pragma unroll
    for (int q = 0; q + w < U; q += 2 * w)
#pragma unroll
      for (int e = 0; e < NV; ++e) acc[q][e] = acc[q][e] + acc[q + w][e];
  if (valid) {
#pragma unroll
    for (int e = 0; e < NV; ++e) store_y(y, k * ldy + j * NV + e, y_f32, acc[0][e]);
  }
}

constexpr int kRowsN = 4;     // rows per wave, F direction
constexpr int kUnrollN = 2;   // vectors per row in flight, F direction
constexpr int kUnrollC = 8;   // rows in flight, F* direction

}  // namespace

hipError_t launch_sbgemv_n(const SbgemvArgs &a, bool compute_f32, hipStream_t s) {
  const int nv = compute_f32 ? 2 : 1;
  const int64_t nvec = (a.Nm + nv - 1) / nv;
  const int64_t ngroups = (a.Nd + kRowsN - 1) / kRowsN;
  const int64_t ntasks = a.K * ngroups;
  const int64_t nblocks = (ntasks + (kBlock / kWave) - 1) / (kBlock / kWave);
  const dim3 grid(static_cast<unsigned>(nblocks)), block(kBlock);
  const int64_t ldF_vec = a.ldF / nv;
  if (compute_f32) {
    hipLaunchKernelGGL((sbgemv_n_kernel<float, float, kRowsN, kUnrollN>), grid, block, 0, s,
                       static_cast<const f32x4 *>(a.F), static_cast<const cx<float> *>(a.x), a.y, a.Nd, ldF_vec,
                       nvec, a.ldx, a.ldy, a.y_f32, ngroups, ntasks, nblocks);
  } else if (a.x_f32) {
    hipLaunchKernelGGL((sbgemv_n_kernel<double, float, kRowsN, kUnrollN>), grid, block, 0, s,
                       static_cast<const f64x2 *>(a.F), static_cast<const cx<float> *>(a.x), a.y, a.Nd, ldF_vec,
                       nvec, a.ldx, a.ldy, a.y_f32, ngroups, ntasks, nblocks);
  } else {
    hipLaunchKernelGGL((sbgemv_n_kernel<double, double, kRowsN, kUnrollN>), grid, block, 0, s,
                       static_cast<const f64x2 *>(a.F), static_cast<const cx<double> *>(a.x), a.y, a.Nd, ldF_vec,
                       nvec, a.ldx, a.ldy, a.y_f32, ngroups, ntasks, nblocks);
  }
  return hipGetLastError();
}

hipError_t launch_sbgemv_c(const SbgemvArgs &a, bool compute_f32, hipStream_t s) {
  const int nv = compute_f32 ? 2 : 1;
  const int64_t nvec = (a.Nm + nv - 1) / nv;
  const int64_t nchunks = (nvec + kBlock - 1) / kBlock;
  const int64_t nblocks = a.K * nchunks;
  const dim3 grid(static_cast<unsigned>(nblocks)), block(kBlock);
  const int64_t ldF_vec = a.ldF / nv;
  if (compute_f32) {
    hipLaunchKernelGGL((sbgemv_c_kernel<float, float, kUnrollC>), grid, block, 0, s,
                       static_cast<const f32x4 *>(a.F), static_cast<const cx<float> *>(a.x), a.y, a.Nd, ldF_vec, nvec,
                       a.ldx, a.ldy, a.y_f32, nchunks, nblocks);
  } else if (a.x_f32) {
    hipLaunchKernelGGL((sbgemv_c_kernel<double, float, kUnrollC>), grid, block, 0, s,
                       static_cast<const f64x2 *>(a.F), static_cast<const cx<float> *>(a.x), a.y, a.Nd, ldF_vec,
                       nvec, a.ldx, a.ldy, a.y_f32, nchunks, nblocks);
  } else {
    hipLaunchKernelGGL((sbgemv_c_kernel<double, double, kUnrollC>), grid, block, 0, s,
                       static_cast<const f64x2 *>(a.F), static_cast<const cx<double> *>(a.x), a.y, a.Nd, ldF_vec,
                       nvec, a.ldx, a.ldy, a.y_f32, nchunks, nblocks);
  }
  return hipGetLastError();
}

}  // namespace fftmv
