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
#include <atomic>

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

// A buffer descriptor over one row (raw: no stride, no swizzle; the fourth
// word is the gfx9 value for untyped 32-bit data). A load through it is the
// row base in scalar registers plus one 32-bit lane offset, so the per-lane
// column offsets are the only address registers a lane keeps, and the
// hardware returns zeros for an offset past the row's end instead of
// reading beyond it.
// The record count is the field's unsigned 32-bit pattern: rows of up to
// 2^31 bytes (Nm <= 2^27 complex128 entries, checked at setup).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void *row, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(row), 0,
                                           static_cast<int32_t>(static_cast<uint32_t>(bytes)), 0x00020000);
}
// 16 bytes at byte_off through a row descriptor, non-temporal (aux bit 1):
// Fhat is read once, and streaming it past the caches keeps the reused
// per-frequency vectors resident.
template <typename V>
__device__ __forceinline__ V load_stream_buf(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(byte_off), 0, 2));
}

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

// The Vec16<T>::n consecutive complex outputs at y[idx..], one store per
// 16 bytes (idx is a multiple of n and rows of y have even length).
template <typename T>
__device__ __forceinline__ void store_vec(void *y, int64_t idx, bool f32, const cx<T> *v) {
  if constexpr (sizeof(T) == 4) {
    if (f32) {
      f32x4 w = {v[0].re, v[0].im, v[1].re, v[1].im};
      *reinterpret_cast<f32x4 *>(static_cast<cx<float> *>(y) + idx) = w;
    } else {
      f64x2 *d = reinterpret_cast<f64x2 *>(static_cast<cx<double> *>(y) + idx);
      d[0] = f64x2{v[0].re, v[0].im};
      d[1] = f64x2{v[1].re, v[1].im};
    }
  } else {
    if (f32)
      static_cast<cx<float> *>(y)[idx] = cvt<float>(v[0]);
    else
      *reinterpret_cast<f64x2 *>(static_cast<cx<double> *>(y) + idx) = f64x2{v[0].re, v[0].im};
  }
}

// 16 bytes at byte_off through a row descriptor, non-temporal (aux bit 1).
// A buffer store with the cache policy as an immediate: a plain pointer
// store chosen by a runtime flag next to it would be merged with it, and
// the non-temporal hint dropped.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
template <typename W>
__device__ __forceinline__ void store_stream_buf(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, W w) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, w), r, static_cast<int>(byte_off), 0, 2);
}

// store_vec through a descriptor of row y_k with non-temporal stores; j is
// the 16-byte input vector index. Not for FP64 sums into FP32 w (8-byte
// stores).
template <typename T>
__device__ __forceinline__ void store_vec_stream(__amdgpu_buffer_rsrc_t r, int64_t j, bool f32, const cx<T> *v) {
  const uint32_t o = static_cast<uint32_t>(j) * 16u;
  if constexpr (sizeof(T) == 4) {
    if (f32) {
      store_stream_buf(r, o, f32x4{v[0].re, v[0].im, v[1].re, v[1].im});
    } else {
      store_stream_buf(r, 2u * o, f64x2{v[0].re, v[0].im});
      store_stream_buf(r, 2u * o + 16u, f64x2{v[1].re, v[1].im});
    }
  } else {
    store_stream_buf(r, o, f64x2{v[0].re, v[0].im});
  }
}

template <typename T>
__device__ __forceinline__ void store_y(void *y, int64_t idx, bool f32, cx<T> v) {
  if (f32)
    static_cast<cx<float> *>(y)[idx] = cvt<float>(v);
  else
    static_cast<cx<double> *>(y)[idx] = cvt<double>(v);
}

// acc += f * x (F) and acc += conj(f) * x (F*), one FMA per real product so
// that each partial sum is a plain FMA chain.
template <typename T>
__device__ __forceinline__ void fma_mul(T &re, T &im, cx<T> f, cx<T> x) {
  re = fma(f.re, x.re, re);
  re = fma(-f.im, x.im, re);
  im = fma(f.re, x.im, im);
  im = fma(f.im, x.re, im);
}
template <typename T>
__device__ __forceinline__ void fma_conj_mul(T &re, T &im, cx<T> f, cx<T> x) {
  re = fma(f.re, x.re, re);
  re = fma(f.im, x.im, re);
  im = fma(f.re, x.im, im);
  im = fma(-f.im, x.re, im);
}

// ------------------------------------------------------------------ F
// v_k[r] = sum_c Fhat_k[r][c] m_k[c].
// One wave per task = (frequency k, R consecutive rows). The wave walks the
// rows side by side: lane l takes 16-byte vectors l, l+64, ... of each row,
// so each load instruction reads 1 KiB contiguous per row, and the matching
// piece of m_k is loaded once for all R rows. U vectors per row are in flight
// per step (R*U Fhat loads issued before any arithmetic). Per-lane partial
// sums are closed with wave_sum (DPP).
template <typename T, typename In, int R, int U, int NCH, int WPE>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void sbgemv_n_kernel(const typename Vec16<T>::type *__restrict__ F,
                                                          const cx<In> *__restrict__ x, void *__restrict__ y,
                                                          int64_t Nd, int64_t ldF_vec, int64_t nvec, int64_t ldx,
                                                          int64_t ldy, bool y_f32, int64_t ngroups, int64_t ntasks,
                                                          int64_t nblocks, cx<T> *__restrict__ part, int64_t ncc,
                                                          int64_t cc_len) {
  using V = typename Vec16<T>::type;
  constexpr int NV = Vec16<T>::n;
  constexpr int NC = U * NV < NCH ? U * NV : NCH;  // chains per row and lane
  const int lane = threadIdx.x & (kWave - 1);
  // the wave index is uniform across the wave: say so, so that the task,
  // the row pointers and the loop bounds live in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t task = xcd_contiguous_block(blockIdx.x, nblocks) * (kBlock / kWave) + wave;
  if (task >= ntasks) return;
  // (frequency, row group), then its column chunk (ncc == 1: whole rows, into y)
  const int64_t kg = ncc == 1 ? task : task / ncc, cc = task - kg * ncc;
  const int64_t k = kg / ngroups;
  const int64_t r0 = (kg - k * ngroups) * R;
  const int64_t c1 = (cc + 1) * cc_len < nvec ? (cc + 1) * cc_len : nvec;

  // one buffer descriptor per row (scalar registers): a load is the row's
  // descriptor plus the lane's 32-bit offset, shared by all R rows
  __amdgpu_buffer_rsrc_t rows[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    int64_t r = r0 + i < Nd ? r0 + i : Nd - 1;  // tail group: re-read the last row, never store it
    rows[i] = row_rsrc(F + (k * Nd + r) * ldF_vec, nvec * static_cast<int64_t>(sizeof(V)));
  }
  const cx<In> *xk = x + k * ldx;

  T ar[R][NC], ai[R][NC];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int c = 0; c < NC; ++c) ar[i][c] = ai[i][c] = T(0);

  int64_t j = cc * cc_len + lane;
  for (; j + (U - 1) * kWave < c1; j += U * kWave) {
    V fv[U][R];
    cx<T> xv[U][NV];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < R; ++i)
        fv[u][i] = load_stream_buf<V>(rows[i], static_cast<uint32_t>(j + u * kWave) * static_cast<uint32_t>(sizeof(V)));
#pragma unroll
    for (int u = 0; u < U; ++u) load_x<T, In>(xk, j + u * kWave, xv[u]);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < R; ++i) {
        cx<T> f[NV];
        split(fv[u][i], f);
#pragma unroll
        for (int e = 0; e < NV; ++e) fma_mul(ar[i][(u * NV + e) % NC], ai[i][(u * NV + e) % NC], f[e], xv[u][e]);
      }
  }
  for (; j < c1; j += kWave) {  // fewer than U vectors left in the chunk
    cx<T> xv[NV];
    load_x<T, In>(xk, j, xv);
#pragma unroll
    for (int i = 0; i < R; ++i) {
      cx<T> f[NV];
      split(load_stream_buf<V>(rows[i], static_cast<uint32_t>(j) * static_cast<uint32_t>(sizeof(V))), f);
#pragma unroll
      for (int e = 0; e < NV; ++e) fma_mul(ar[i][e % NC], ai[i][e % NC], f[e], xv[e]);
    }
  }

#pragma unroll
  for (int i = 0; i < R; ++i) {
    // pairwise tree over this lane's chains, then across the wave
#pragma unroll
    for (int w = 1; w < NC; w *= 2)
#pragma unroll
      for (int q = 0; q + w < NC; q += 2 * w) {
        ar[i][q] += ar[i][q + w];
        ai[i][q] += ai[i][q + w];
      }
    cx<T> s = mk(wave_sum(ar[i][0]), wave_sum(ai[i][0]));
    if (lane == 0 && r0 + i < Nd) {
      if (ncc == 1)
        store_y(y, k * ldy + r0 + i, y_f32, s);
      else
        part[(k * ncc + cc) * Nd + r0 + i] = s;
    }
  }
}

// Column-chunk sums of the wide-row F kernel, in chunk order, into v_k.
template <typename T>
__global__ __launch_bounds__(kBlock) void sbgemv_n_reduce_kernel(const cx<T> *__restrict__ part, void *y, int64_t K,
                                                                 int64_t Nd, int64_t ncc, int64_t ldy, bool y_f32) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (i >= K * Nd) return;
  const int64_t k = i / Nd, r = i - k * Nd;
  cx<T> acc = part[(k * ncc) * Nd + r];
  for (int64_t c = 1; c < ncc; ++c) {
    const cx<T> v = part[(k * ncc + c) * Nd + r];
    acc = mk(acc.re + v.re, acc.im + v.im);
  }
  store_y(y, k * ldy + r, y_f32, acc);
}

// ------------------------------------------------------------- F, whole rows
// v_k[r] = sum_c Fhat_k[r][c] m_k[c] with one workgroup of TPB threads per
// frequency (FP32): lane t holds m_k's vectors t, t + TPB, ... (VL of them)
// in registers, and the workgroup walks the rows of F̂_k one at a time, all
// lanes reading one row together, so each workgroup streams its frequency
// block front to back. Per row each lane adds its VL vector products in one
// chain, each wave closes its partial with wave_sum (DPP) into LDS
// ([Nd][waves], Nd * waves * 8 bytes), and after the last row the waves'
// partials of each row are added in wave order: fixed orders throughout.
template <typename In, int TPB, int VL>
__global__ __launch_bounds__(TPB) __attribute__((amdgpu_waves_per_eu(8, 8))) void sbgemv_n_row_kernel(
    const f32x4 *__restrict__ F, const cx<In> *__restrict__ x, void *__restrict__ y, int64_t Nd, int64_t ldF_vec,
    int64_t nvec, int64_t ldx, int64_t ldy, bool y_f32, int64_t nblocks) {
  using T = float;
  constexpr int W = TPB / kWave;
  extern __shared__ __align__(16) unsigned char smem[];
  cx<T> *red = reinterpret_cast<cx<T> *>(smem);
  const int64_t k = xcd_contiguous_block(blockIdx.x, nblocks);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const f32x4 *base = F + k * Nd * ldF_vec;
  cx<T> xv[VL][2];
#pragma unroll
  for (int v = 0; v < VL; ++v) {
    const int64_t j = threadIdx.x + static_cast<int64_t>(v) * TPB;
    if (j < nvec) {
      load_x<T, In>(x + k * ldx, j, xv[v]);
    } else {  // past the end: the clamped loads below add nothing
      xv[v][0] = mk(T(0), T(0));
      xv[v][1] = mk(T(0), T(0));
    }
  }
  const uint32_t off0 = threadIdx.x * 16u, last = static_cast<uint32_t>(nvec - 1) * 16u;
  const int64_t row_bytes = nvec * 16;
  for (int64_t r = 0; r < Nd; ++r) {
    const __amdgpu_buffer_rsrc_t rs = row_rsrc(base + r * ldF_vec, row_bytes);
    T re = T(0), im = T(0);
#pragma unroll
    for (int v = 0; v < VL; ++v) {
      uint32_t o = off0 + static_cast<uint32_t>(v * TPB * 16);
      o = o < last ? o : last;
      cx<T> f[2];
      split(load_stream_buf<f32x4>(rs, o), f);
#pragma unroll
      for (int e = 0; e < 2; ++e) fma_mul(re, im, f[e], xv[v][e]);
      __builtin_amdgcn_sched_barrier(0);  // one load in flight per wave
    }
    re = wave_sum(re);
    im = wave_sum(im);
    if (lane == 0) red[r * W + wave] = mk(re, im);
  }
  __syncthreads();
  for (int64_t r = threadIdx.x; r < Nd; r += TPB) {
    cx<T> sum = red[r * W];
#pragma unroll
    for (int w = 1; w < W; ++w) sum = sum + red[r * W + w];
    store_y(y, k * ldy + r, y_f32, sum);
  }
}

// ----------------------------------------------------------- F, narrow rows
// v_k[r] = sum_c Fhat_k[r][c] m_k[c] when rows have at most 32 16-byte
// vectors: the wave-per-four-rows kernel would leave most lanes idle. Thread
// t takes column vector j = t % G of row slot q = t / G (G the power of two
// >= nvec, P = 256 / G row slots per workgroup), keeps m_k's vector j in
// registers and walks rows q, q + P, ... of its workgroup's row segment; the
// G lanes of a row add their products with a butterfly in a fixed order.
template <typename T, typename In, int G>
__global__ __launch_bounds__(kBlock) void sbgemv_n_narrow_kernel(const typename Vec16<T>::type *__restrict__ F,
                                                                 const cx<In> *__restrict__ x, void *__restrict__ y,
                                                                 int64_t Nd, int64_t ldF_vec, int64_t nvec,
                                                                 int64_t ldx, int64_t ldy, bool y_f32, int64_t nseg,
                                                                 int64_t seg_rows, int64_t nblocks) {
  using V = typename Vec16<T>::type;
  constexpr int NV = Vec16<T>::n;
  constexpr int P = kBlock / G;
  const int64_t blk = xcd_contiguous_block(blockIdx.x, nblocks);
  const int64_t k = blk / nseg, seg = blk - k * nseg;
  const int t = threadIdx.x, q = t / G, j = t % G;
  const bool live = j < nvec;
  cx<T> xv[NV];
#pragma unroll
  for (int e = 0; e < NV; ++e) xv[e] = mk(T(0), T(0));
  if (live) load_x<T, In>(x + k * ldx, j, xv);
  const int64_t r1 = (seg + 1) * seg_rows < Nd ? (seg + 1) * seg_rows : Nd;
  const V *col = F + k * Nd * ldF_vec + (live ? j : 0);
  auto row = [&](int64_t r) {
    T re = T(0), im = T(0);
    if (live) {
      cx<T> f[NV];
      split(__builtin_nontemporal_load(col + r * ldF_vec), f);
#pragma unroll
      for (int e = 0; e < NV; ++e) fma_mul(re, im, f[e], xv[e]);
    }
#pragma unroll
    for (int m = 1; m < G; m <<= 1) {
      re += __shfl_xor(re, m);
      im += __shfl_xor(im, m);
    }
    if (j == 0) store_y(y, k * ldy + r, y_f32, mk(re, im));
  };
  // the G lanes of one row share q, so they run the same iterations; with
  // G > 1 the rows' cross-lane exchanges keep the compiler from unrolling a
  // loop whose trip count is known only at run time
  const int64_t r0 = seg * seg_rows + q;
  if constexpr (G == 1) {
#pragma unroll 4
    for (int64_t r = r0; r < r1; r += P) row(r);
  } else {
    for (int64_t r = r0; r < r1; r += P) row(r);
  }
}

// ------------------------------------------------------------------ F*
// w_k[c] = sum_r conj(Fhat_k[r][c]) d_k[r].
// One workgroup of TPB threads per (frequency k, chunk of VL*TPB consecutive
// 16-byte column vectors): each lane owns VL vectors TPB apart (a vector is
// two complex64 columns or one complex128 column) and walks down all Nd
// rows in steps of U rows, keeping one partial sum per column: no
// cross-lane reduction. The U products of a step are added together before
// they enter the column's sum, so that in FP32 no chain is longer than
// about Nd / U additions (one chain over all Nd rows costs 2.3x the error at
// Nd = 100). That fits a lane in 64 VGPRs, so eight waves run
// per SIMD and every workgroup of the Main shape (one 512-thread chunk per
// frequency: 1001 workgroups on 1024 slots) is resident at once; with the
// offsets formed at each load, 10 vectors per lane still fit. Each wave
// keeps ONE 16-byte load in flight and waits for it before the next.
// Measured at Main with two 256-thread chunks per frequency: that (600 us, with
// the loads through a row buffer descriptor; 604 us with 64-bit addresses,
// which spill at 64 VGPRs) beats all VL loads of a row in flight (650 us),
// two rows per load group at four waves per SIMD (622 us), two partial sums
// per column (641 us, spills) and the rows split over two half-workgroups
// (630 us). d_k[r] is the same for the whole workgroup (a scalar load, U
// rows per load). TPB is 256, or 384 / 512 / 1024 for rows that one
// workgroup covers whole (see choose_chunks_c). nt_y: w is written with
// non-temporal stores (large outputs, see kStreamOutBytesC).
template <typename T, typename In, int VL, int U, int TPB>
__global__ __launch_bounds__(TPB) __attribute__((amdgpu_waves_per_eu(8, 8))) void sbgemv_c_kernel(
    const typename Vec16<T>::type *__restrict__ F, const cx<In> *__restrict__ x, void *__restrict__ y, int64_t Nd,
    int64_t ldF_vec, int64_t nvec, int64_t ldx, int64_t ldy, bool y_f32, int64_t nchunks, int64_t nblocks,
    cx<T> *__restrict__ part, int64_t nseg, int64_t seg_rows, bool nt_y) {
  using V = typename Vec16<T>::type;
  constexpr int NV = Vec16<T>::n;
  const int64_t blk = xcd_contiguous_block(blockIdx.x, nblocks);
  // tile (k, chunk), then its row segment (nseg == 1: all Nd rows, into y)
  const int64_t tile = nseg == 1 ? blk : blk / nseg, seg = blk - tile * nseg;
  const int64_t k = tile / nchunks;
  const int64_t j0 = (tile - k * nchunks) * (TPB * VL) + threadIdx.x;
  const int64_t r_end = (seg + 1) * seg_rows < Nd ? (seg + 1) * seg_rows : Nd;
  const V *base = F + k * Nd * ldF_vec;
  const cx<In> *xk = x + k * ldx;
  // byte offset of vector v of this lane within a row (rows are far below
  // 4 GiB), formed at each load instead of held in VL registers; lanes past
  // the end re-read the last vector and never store
  const uint32_t off0 = static_cast<uint32_t>(j0) * static_cast<uint32_t>(sizeof(V));
  const uint32_t last = static_cast<uint32_t>(nvec - 1) * static_cast<uint32_t>(sizeof(V));
  auto off = [&](int v) {
    const uint32_t o = off0 + static_cast<uint32_t>(v * TPB * static_cast<int>(sizeof(V)));
    return o < last ? o : last;
  };

  T ar[VL][NV], ai[VL][NV];
#pragma unroll
  for (int v = 0; v < VL; ++v)
#pragma unroll
    for (int e = 0; e < NV; ++e) ar[v][e] = ai[v][e] = T(0);

  const int64_t row_bytes = nvec * static_cast<int64_t>(sizeof(V));
  int64_t r = seg * seg_rows;
  for (; r + U <= r_end; r += U) {
    cx<T> d[U];
#pragma unroll
    for (int u = 0; u < U; ++u) d[u] = cvt<T>(xk[r + u]);
    if constexpr (sizeof(T) == 4) {
      // FP32: the U rows' products of each column are summed first and
      // enter the column's sum once, so the chains are U and Nd / U
      // additions long instead of one of Nd
      __amdgpu_buffer_rsrc_t rs[U];
#pragma unroll
      for (int u = 0; u < U; ++u) rs[u] = row_rsrc(base + (r + u) * ldF_vec, row_bytes);
#pragma unroll
      for (int v = 0; v < VL; ++v) {
        T gr[NV], gi[NV];
#pragma unroll
        for (int e = 0; e < NV; ++e) gr[e] = gi[e] = T(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          cx<T> f[NV];
          split(load_stream_buf<V>(rs[u], off(v)), f);
#pragma unroll
          for (int e = 0; e < NV; ++e) fma_conj_mul(gr[e], gi[e], f[e], d[u]);
          __builtin_amdgcn_sched_barrier(0);  // one load in flight per wave
        }
#pragma unroll
        for (int e = 0; e < NV; ++e) {
          ar[v][e] += gr[e];
          ai[v][e] += gi[e];
        }
      }
    } else {
      // FP64: rows added to the column sums one by one (the chain length
      // is far below the FP64 error budget; the row step keeps the
      // registers of the longest rows without spills)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const __amdgpu_buffer_rsrc_t rs = row_rsrc(base + (r + u) * ldF_vec, row_bytes);
#pragma unroll
        for (int v = 0; v < VL; ++v) {
          cx<T> f[NV];
          split(load_stream_buf<V>(rs, off(v)), f);
#pragma unroll
          for (int e = 0; e < NV; ++e) fma_conj_mul(ar[v][e], ai[v][e], f[e], d[u]);
          __builtin_amdgcn_sched_barrier(0);  // one load in flight per wave
        }
      }
    }
  }
  for (; r < r_end; ++r) {  // fewer than U rows left
    const cx<T> d = cvt<T>(xk[r]);
    const __amdgpu_buffer_rsrc_t rs = row_rsrc(base + r * ldF_vec, row_bytes);
#pragma unroll
    for (int v = 0; v < VL; ++v) {
      cx<T> f[NV];
      split(load_stream_buf<V>(rs, off(v)), f);
#pragma unroll
      for (int e = 0; e < NV; ++e) fma_conj_mul(ar[v][e], ai[v][e], f[e], d);
    }
  }

  // row y_k for non-temporal stores: nvec * NV complex entries
  const __amdgpu_buffer_rsrc_t yrs =
      y_f32 ? row_rsrc(static_cast<cx<float> *>(y) + k * ldy, nvec * NV * 8)
            : row_rsrc(static_cast<cx<double> *>(y) + k * ldy, nvec * NV * 16);
#pragma unroll
  for (int v = 0; v < VL; ++v) {
    const int64_t j = j0 + v * TPB;
    if (j < nvec) {
      cx<T> out[NV];
#pragma unroll
      for (int e = 0; e < NV; ++e) out[e] = mk(ar[v][e], ai[v][e]);
      if (nseg == 1) {
        if (nt_y)
          store_vec_stream(yrs, j, y_f32, out);
        else
          store_vec(y, k * ldy + j * NV, y_f32, out);
      } else {
#pragma unroll
        for (int e = 0; e < NV; ++e) part[((k * nseg + seg) * nvec + j) * NV + e] = out[e];
      }
    }
  }
}

// ------------------------------------------------------- F*, tall blocks
// w_k[c] = sum_r conj(Fhat_k[r][c]) d_k[r] when a block has few columns
// (nvec <= 128 16-byte vectors) and many rows: the short-wide kernel would
// leave most lanes idle and walk all Nd rows one load at a time. Here thread
// t of a workgroup takes column vector j = t % nvec and rows q, q + P, ...
// (q = t / nvec, P = 256 / nvec rows per step) of one segment of rows, so a
// step loads P rows x nvec vectors; the P partial sums of each column are
// added in LDS in row-slot order and written per (frequency, segment); a
// second kernel adds the segments in order. Fixed orders throughout, so the
// result is bitwise repeatable.
template <typename T, typename In>
__global__ __launch_bounds__(kBlock) void sbgemv_c_tall_kernel(const typename Vec16<T>::type *__restrict__ F,
                                                               const cx<In> *__restrict__ x, cx<T> *__restrict__ part,
                                                               int64_t Nd, int64_t ldF_vec, int64_t nvec, int64_t ldx,
                                                               int64_t nseg, int64_t seg_rows, int64_t nblocks) {
  using V = typename Vec16<T>::type;
  constexpr int NV = Vec16<T>::n;
  __shared__ cx<T> red[kBlock * NV];
  const int64_t blk = xcd_contiguous_block(blockIdx.x, nblocks);
  const int64_t k = blk / nseg, seg = blk - k * nseg;
  const int nv = static_cast<int>(nvec);
  const int P = kBlock / nv;
  const int t = threadIdx.x, q = t / nv, j = t - q * nv;
  T ar[NV], ai[NV];
#pragma unroll
  for (int e = 0; e < NV; ++e) ar[e] = ai[e] = T(0);
  if (q < P) {
    const int64_t r1 = (seg + 1) * seg_rows < Nd ? (seg + 1) * seg_rows : Nd;
    const V *col = F + k * Nd * ldF_vec + j;
    const cx<In> *xk = x + k * ldx;
#pragma unroll 4
    for (int64_t r = seg * seg_rows + q; r < r1; r += P) {
      const cx<T> d = cvt<T>(xk[r]);
      cx<T> f[NV];
      split(__builtin_nontemporal_load(col + r * ldF_vec), f);
#pragma unroll
      for (int e = 0; e < NV; ++e) fma_conj_mul(ar[e], ai[e], f[e], d);
    }
  }
#pragma unroll
  for (int e = 0; e < NV; ++e) red[t * NV + e] = mk(ar[e], ai[e]);
  __syncthreads();
  if (t < nv) {
    cx<T> acc[NV];
#pragma unroll
    for (int e = 0; e < NV; ++e) acc[e] = red[t * NV + e];
    for (int qq = 1; qq < P; ++qq)
#pragma unroll
      for (int e = 0; e < NV; ++e) {
        const cx<T> v = red[(qq * nv + t) * NV + e];
        acc[e] = mk(acc[e].re + v.re, acc[e].im + v.im);
      }
#pragma unroll
    for (int e = 0; e < NV; ++e) part[((k * nseg + seg) * nvec + t) * NV + e] = acc[e];
  }
}

// Segment sums (tall-block form, or row segments of the short-wide kernel),
// in segment order, into w_k.
template <typename T>
__global__ __launch_bounds__(kBlock) void sbgemv_c_reduce_kernel(const cx<T> *__restrict__ part, void *y,
                                                                      int64_t K, int64_t nseg, int64_t nvec,
                                                                      int64_t ldy, bool y_f32) {
  constexpr int NV = Vec16<T>::n;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (i >= K * nvec) return;
  const int64_t k = i / nvec, j = i - k * nvec;
  cx<T> acc[NV];
#pragma unroll
  for (int e = 0; e < NV; ++e) acc[e] = part[((k * nseg) * nvec + j) * NV + e];
  for (int64_t sg = 1; sg < nseg; ++sg)
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      const cx<T> v = part[((k * nseg + sg) * nvec + j) * NV + e];
      acc[e] = mk(acc[e].re + v.re, acc[e].im + v.im);
    }
  store_vec(y, k * ldy + j * NV, y_f32, acc);
}

constexpr int kRowsN = 4;    // rows per wave, F direction
constexpr int kUnrollN = 2;  // vectors per row in flight, F direction
constexpr int kChainsN = 4;  // partial sums per row and lane, F direction
constexpr int kWavesN = 4;   // waves per SIMD the registers are sized for, F direction
constexpr int kMaxVecsC = 5;  // vectors per lane, F* direction (at most)
// Rows per step of the conjugate-transpose kernel (F* direction): one scalar
// load of d_k per row; in FP32 the step's products of each column are
// summed before they enter the column's sum. Measured at Nm=5000, Nd=100,
// Nt=1000 (FP32, 512-thread whole rows): F* error of the FP32 SBGEMV alone
// 1.94e-7 with every row added to the column sum directly, 1.07e-7 in steps
// of 2 rows, 8.6e-8 of 4, 8.3e-8 of 5; kernel time 588, 590, 592, 592 us.
// FP64 keeps steps of 2 (five rows of complex128 d_k spill the widest rows),
// and so does FP32 at 8 vectors per lane (5 and 4 rows spill 2 VGPRs there).
template <typename T, int VL>
constexpr int unroll_c() { return sizeof(T) == 4 && VL != 8 ? 5 : 2; }

// Output size (bytes of w over all frequencies) from which the conjugate-
// transpose kernel stores w with non-temporal stores (not FP64 sums into
// FP32 w, whose stores are 8 bytes). Measured for FP32 w at
// K = 2001, Nd = 100, whole-row workgroups of 1024 threads: from 128 MB of
// output (Nm = 8000) to 320 MB (Nm = 20000) the kernel runs 5-7% faster
// with them (4.88 against 5.22 ms at Nm = 20000); the end-of-workgroup store
// burst through the caches otherwise costs about 10% of the kernel (4.55 ms
// with the stores left out). At Nm = 5000, K = 1001 (40 MB) they gain
// nothing (638 against 636 us), and an output that fits the last-level
// cache can be read from there by the inverse FFT that follows.
constexpr int64_t kStreamOutBytesC = int64_t(64) << 20;

template <typename T, typename In, int VL, int TPB>
hipError_t launch_c(const SbgemvArgs &a, int64_t nvec, int64_t nchunks, int64_t nseg, int64_t seg_rows,
                    hipStream_t s) {
  using V = typename Vec16<T>::type;
  const int nv = Vec16<T>::n;
  const int64_t nblocks = a.K * nchunks * nseg;
  const int64_t nred = (a.K * nvec + kBlock - 1) / kBlock;
  if (!grid_fits(nblocks, TPB) || !grid_fits(nred, kBlock)) return hipErrorInvalidConfiguration;
  cx<T> *part = static_cast<cx<T> *>(a.part);
  const bool nt_y = nseg == 1 && !(sizeof(T) == 8 && a.y_f32) &&
                    a.K * a.ldy * (a.y_f32 ? 8 : 16) >= kStreamOutBytesC;
  hipLaunchKernelGGL((sbgemv_c_kernel<T, In, VL, unroll_c<T, VL>(), TPB>), dim3(static_cast<unsigned>(nblocks)),
                     dim3(TPB), 0, s, static_cast<const V *>(a.F), static_cast<const cx<In> *>(a.x), a.y, a.Nd,
                     a.ldF / nv, nvec, a.ldx, a.ldy, a.y_f32, nchunks, nblocks, part, nseg, seg_rows, nt_y);
  if (nseg > 1) {
    hipLaunchKernelGGL((sbgemv_c_reduce_kernel<T>), dim3(static_cast<unsigned>(nred)), dim3(kBlock), 0, s, part,
                       a.y, a.K, nseg, nvec, a.ldy, a.y_f32);
  }
  return hipSuccess;
}

// Workgroups of the conjugate-transpose kernel that one CU holds at once:
// 64 VGPRs and no LDS give eight waves on each of four SIMDs, four waves per
// workgroup.
constexpr int kResidentPerCuC = 8;
// A narrower column chunk is taken only when it fills the rounds of
// resident workgroups better than the current pick by more than this.
constexpr double kFillMargin = 0.05;

int resident_c_workgroups() {
  static std::atomic<int> cus_of[64];  // per device, 0 until queried
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (dev >= 0 && dev < 64) cus = cus_of[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (dev >= 0 && dev < 64) cus_of[dev].store(cus, std::memory_order_relaxed);
  }
  return kResidentPerCuC * cus;
}

struct ChunksC {
  int64_t vl = 1, nchunks = 1;
  int tpb = kBlock;  // threads per workgroup
};

// Workgroup sizes of the whole-row form (see choose_chunks_c), each with
// the vectors per lane it takes: at most 10 in FP32 (60 VGPRs) and 7 in
// FP64, whose kernels spill registers from 8 vectors per lane; at least
// enough that few lanes idle.
struct RowFormC {
  int tpb;
  int64_t vl_min, vl_max32, vl_max64;
};
constexpr RowFormC kRowFormsC[] = {{1024, 3, 10, 7}, {512, 3, 5, 5}, {384, 4, 7, 7}};
template <typename T>
constexpr int64_t max_vecs_row_c() {
  return sizeof(T) == 4 ? 10 : 7;
}
// resident workgroups of tpb threads, from those of 256 (eight waves per
// SIMD either way)
int64_t slots_for(int64_t slots256, int tpb) {
  return slots256 / kResidentPerCuC * (int64_t(kResidentPerCuC) * kBlock / tpb);
}

// Column chunks of one frequency for the conjugate-transpose kernel. A
// workgroup holds its chunk for all Nd rows with one load in flight per
// wave, so a launch that overflows the resident workgroups by a few leaves
// those few to run almost alone at the end: at Nm = 5000, Nt = 1029 (1030
// frequencies) two chunks per frequency make 2060 workgroups on 2048 slots
// and take 808 us, five chunks (2 vectors per lane, 5150 workgroups, the
// last round 51% full) 669 us. For each width of 5 down to 1 vectors per
// lane (then the fewest, equal chunks that cover the row) this takes the
// fill of the rounds, workgroups / (rounds x slots), and keeps the widest
// chunk unless a narrower one fills clearly better (the Main and Scale
// shapes would keep 5 vectors per lane, fill 0.978 and 0.977, but take the
// whole-row form below).
// Rows that 256 threads cannot cover at 5 vectors per lane go whole to one
// workgroup of 1024, 512 or 384 threads (kRowFormsC; up to 10240
// vectors, 7168 in FP64): each workgroup then streams its frequency block
// front to back instead of sharing every row with other workgroups. Of the
// sizes whose vectors per lane fit the row, the one that fills its rounds
// of resident slots best is taken (on a tie, the one with fewer idle
// lanes), and it is used unless the 256-thread chunks fill clearly better
// (by more than kFillMargin): a row streamed whole in one round beats
// chunks that need several. Measured on one box against the 256-thread
// chunks: Main (2500 vectors, 512 x 5) 621 -> 604 us; 1030 frequencies of
// 2500 vectors (Nt = 1029; 384 x 7, one round of 1280 slots where 512
// threads would need two) 689 -> 645 us; 1200 frequencies 799 -> 734 us;
// Nm = 10000 (5000 vectors, 1024 x 5) 1235 -> 1221 us; the Scale share
// (10000 vectors, 1024 x 10) 5419 -> 5086 us. Rows cut into two or more
// such chunks measured no faster than the 256-thread form, which longer
// rows keep. A whole-row launch with a thin last round is slow (its last
// workgroups stream whole blocks almost alone): 1401 frequencies in
// 320-thread workgroups took 1131 us against 881 us in 256-thread chunks,
// so 320 threads (five waves, whose workgroups did not all stay resident)
// are not among the sizes.
ChunksC choose_chunks_c(int64_t K, int64_t nvec, int64_t slots, bool f32) {
  ChunksC best;
  double best_fill = -1.0;
  for (int64_t m = kMaxVecsC; m >= 1; --m) {
    const int64_t nch0 = (nvec + kBlock * m - 1) / (kBlock * m);
    const int64_t vl = (nvec + nch0 * kBlock - 1) / (nch0 * kBlock);
    const int64_t nch = (nvec + vl * kBlock - 1) / (vl * kBlock);
    const int64_t n = K * nch;
    const int64_t rounds = (n + slots - 1) / slots;
    const double fill = static_cast<double>(n) / static_cast<double>(rounds * slots);
    if (fill > best_fill + kFillMargin) {
      best = {vl, nch, kBlock};
      best_fill = fill;
    }
  }
  if (nvec <= int64_t(kBlock) * kMaxVecsC) return best;
  ChunksC row;
  double row_fill = -1.0, row_busy = 0.0;
  for (const RowFormC &f : kRowFormsC) {
    const int64_t vl = (nvec + f.tpb - 1) / f.tpb;
    if (vl < f.vl_min || vl > (f32 ? f.vl_max32 : f.vl_max64)) continue;
    const int64_t s2 = slots_for(slots, f.tpb);
    const int64_t rounds = (K + s2 - 1) / s2;
    const double fill = static_cast<double>(K) / static_cast<double>(rounds * s2);
    const double busy = static_cast<double>(nvec) / static_cast<double>(vl * f.tpb);
    if (fill > row_fill + 1e-9 || (fill > row_fill - 1e-9 && busy > row_busy)) {
      row = {vl, 1, f.tpb};
      row_fill = fill;
      row_busy = busy;
    }
  }
  if (row_fill >= 0 && row_fill + kFillMargin >= best_fill) best = row;
  return best;
}

// Row segments of the short-wide kernel: when its tiles fill less than half
// a round of resident workgroups, each tile walks all Nd rows one load at a
// time while most of the GPU idles (few frequencies and many rows, e.g.
// Nt = 256 with Nd = 4000). The rows are then split into nseg segments (at
// most slots / tiles of them, at least kSegMinRows rows each); each
// workgroup stores its segment's partial sums in the plan workspace and a
// second kernel adds the segments in order.
constexpr int64_t kSegMinRows = 32;
// Segments are also at most kSegMaxRows long, which bounds the FP32 chain
// of a column sum to about kSegMaxRows / 5 additions in FP32 (Nm = 600, Nd = 4000,
// Nt = 256 in 3 segments of 1334 rows, every row added to the column sum
// directly: F* error 7.4e-7 of the 1e-6 budget).
constexpr int64_t kSegMaxRows = 512;

struct SegC {
  int64_t nseg = 1, seg_rows = 0;
};

// slots: resident 256-thread workgroups; a chunking of c.tpb threads has
// slots * 256 / c.tpb of them.
SegC seg_c(int64_t K, const ChunksC &c, int64_t Nd, int64_t slots) {
  SegC sc;
  sc.seg_rows = Nd;
  int64_t n = slots_for(slots, c.tpb) / (K * c.nchunks);
  const int64_t by_rows = Nd / kSegMinRows;
  n = n < by_rows ? n : by_rows;
  const int64_t by_chain = (Nd + kSegMaxRows - 1) / kSegMaxRows;
  n = n > by_chain ? n : by_chain;
  if (n < 2) return sc;
  sc.seg_rows = (Nd + n - 1) / n;
  sc.nseg = (Nd + sc.seg_rows - 1) / sc.seg_rows;
  return sc;
}

size_t seg_part_bytes(int64_t K, int64_t nvec, const SegC &sc) {
  return sc.nseg > 1 ? static_cast<size_t>(K * sc.nseg * nvec) * 16 : 0;
}

// the whole-row launch of c.vl vectors per lane, VL..VLMAX
template <typename T, typename In, int TPB, int VL, int VLMAX>
hipError_t launch_row_c(const SbgemvArgs &a, int64_t nvec, const ChunksC &c, const SegC &sc, hipStream_t s) {
  if constexpr (VL > VLMAX) {
    return hipErrorInvalidValue;  // not reached: choose_chunks_c keeps vl within the form's range
  } else {
    if (c.vl == VL) return launch_c<T, In, VL, TPB>(a, nvec, c.nchunks, sc.nseg, sc.seg_rows, s);
    return launch_row_c<T, In, TPB, VL + 1, VLMAX>(a, nvec, c, sc, s);
  }
}

template <typename T, typename In>
hipError_t launch_c_vl(const SbgemvArgs &a, int64_t nvec, hipStream_t s) {
  const int64_t slots = resident_c_workgroups();
  const ChunksC c = choose_chunks_c(a.K, nvec, slots, sizeof(T) == 4);
  SegC sc = seg_c(a.K, c, a.Nd, slots);
  if (sc.nseg > 1 && !(a.part && a.part_bytes >= seg_part_bytes(a.K, nvec, sc))) {
    sc.nseg = 1;  // no workspace (callers outside an apply): all rows in one pass
    sc.seg_rows = a.Nd;
  }
  constexpr int64_t cap = max_vecs_row_c<T>();
  switch (c.tpb) {
    case 1024: return launch_row_c<T, In, 1024, 3, cap>(a, nvec, c, sc, s);
    case 512: return launch_row_c<T, In, 512, 3, 5>(a, nvec, c, sc, s);
    case 384: return launch_row_c<T, In, 384, 4, 7>(a, nvec, c, sc, s);
    default: break;
  }
  switch (c.vl) {
    case 1: return launch_c<T, In, 1, kBlock>(a, nvec, c.nchunks, sc.nseg, sc.seg_rows, s);
    case 2: return launch_c<T, In, 2, kBlock>(a, nvec, c.nchunks, sc.nseg, sc.seg_rows, s);
    case 3: return launch_c<T, In, 3, kBlock>(a, nvec, c.nchunks, sc.nseg, sc.seg_rows, s);
    case 4: return launch_c<T, In, 4, kBlock>(a, nvec, c.nchunks, sc.nseg, sc.seg_rows, s);
    default: return launch_c<T, In, 5, kBlock>(a, nvec, c.nchunks, sc.nseg, sc.seg_rows, s);
  }
}

// The tall-block form of F*: used when a block has at most 128 column
// vectors (two rows per step at least) and at least kTallMinRows rows.
// Segments of rows give at least kTallMinBlocks workgroups when the rows
// allow it, each thread keeping at least kTallMinPerThread rows.
constexpr int64_t kTallMaxVecs = kBlock / 2;
constexpr int64_t kTallMinRows = 64;
constexpr int64_t kTallMinBlocks = 4096;
constexpr int64_t kTallMinPerThread = 8;

struct TallSplit {
  int64_t nseg = 0, seg_rows = 0;  // nseg == 0: not the tall-block form
};

TallSplit tall_split(int64_t K, int64_t Nd, int64_t nvec) {
  TallSplit ts;
  if (nvec > kTallMaxVecs || Nd < kTallMinRows || K < 1) return ts;
  const int64_t P = kBlock / nvec;
  int64_t max_seg = Nd / (P * kTallMinPerThread);
  max_seg = max_seg < 1 ? 1 : max_seg;
  int64_t want = (kTallMinBlocks + K - 1) / K;
  want = want < 1 ? 1 : want;
  const int64_t nseg0 = want < max_seg ? want : max_seg;
  ts.seg_rows = (Nd + nseg0 - 1) / nseg0;
  ts.nseg = (Nd + ts.seg_rows - 1) / ts.seg_rows;
  return ts;
}

size_t tall_part_bytes(int64_t K, int64_t nvec, const TallSplit &ts) {
  return static_cast<size_t>(K * ts.nseg * nvec) * 16;  // one 16-byte vector per (k, segment, column vector)
}

template <typename T, typename In>
hipError_t launch_c_tall(const SbgemvArgs &a, int64_t nvec, const TallSplit &ts, hipStream_t s) {
  using V = typename Vec16<T>::type;
  const int nv = Vec16<T>::n;
  const int64_t nblocks = a.K * ts.nseg;
  const int64_t nred = (a.K * nvec + kBlock - 1) / kBlock;
  if (!grid_fits(nblocks, kBlock) || !grid_fits(nred, kBlock)) return hipErrorInvalidConfiguration;
  cx<T> *part = static_cast<cx<T> *>(a.part);
  hipLaunchKernelGGL((sbgemv_c_tall_kernel<T, In>), dim3(static_cast<unsigned>(nblocks)), dim3(kBlock), 0, s,
                     static_cast<const V *>(a.F), static_cast<const cx<In> *>(a.x), part, a.Nd, a.ldF / nv, nvec,
                     a.ldx, ts.nseg, ts.seg_rows, nblocks);
  hipLaunchKernelGGL((sbgemv_c_reduce_kernel<T>), dim3(static_cast<unsigned>(nred)), dim3(kBlock), 0, s, part,
                     a.y, a.K, ts.nseg, nvec, a.ldy, a.y_f32);
  return hipSuccess;
}

// The narrow-row form of F: rows of at most kNarrowMaxVecs vectors, in
// segments that give at least kTallMinBlocks workgroups when the rows allow
// it, each thread keeping at least kTallMinPerThread rows.
constexpr int64_t kNarrowMaxVecs = 32;

struct NarrowSplit {
  int G = 0;  // 0: not the narrow-row form
  int64_t nseg = 0, seg_rows = 0;
};

NarrowSplit narrow_split(int64_t K, int64_t Nd, int64_t nvec) {
  NarrowSplit ns;
  if (nvec > kNarrowMaxVecs || K < 1 || Nd < 1) return ns;
  int G = 1;
  while (G < nvec) G <<= 1;
  const int64_t P = kBlock / G;
  int64_t max_seg = Nd / (P * kTallMinPerThread);
  max_seg = max_seg < 1 ? 1 : max_seg;
  int64_t want = (kTallMinBlocks + K - 1) / K;
  want = want < 1 ? 1 : want;
  const int64_t nseg0 = want < max_seg ? want : max_seg;
  ns.G = G;
  ns.seg_rows = (Nd + nseg0 - 1) / nseg0;
  ns.nseg = (Nd + ns.seg_rows - 1) / ns.seg_rows;
  return ns;
}

template <typename T, typename In, int G>
hipError_t launch_n_narrow_g(const SbgemvArgs &a, int64_t nvec, const NarrowSplit &ns, hipStream_t s) {
  using V = typename Vec16<T>::type;
  const int nv = Vec16<T>::n;
  const int64_t nblocks = a.K * ns.nseg;
  if (!grid_fits(nblocks, kBlock)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((sbgemv_n_narrow_kernel<T, In, G>), dim3(static_cast<unsigned>(nblocks)), dim3(kBlock), 0, s,
                     static_cast<const V *>(a.F), static_cast<const cx<In> *>(a.x), a.y, a.Nd, a.ldF / nv, nvec,
                     a.ldx, a.ldy, a.y_f32, ns.nseg, ns.seg_rows, nblocks);
  return hipSuccess;
}

template <typename T, typename In>
hipError_t launch_n_narrow(const SbgemvArgs &a, int64_t nvec, const NarrowSplit &ns, hipStream_t s) {
  switch (ns.G) {
    case 1: return launch_n_narrow_g<T, In, 1>(a, nvec, ns, s);
    case 2: return launch_n_narrow_g<T, In, 2>(a, nvec, ns, s);
    case 4: return launch_n_narrow_g<T, In, 4>(a, nvec, ns, s);
    case 8: return launch_n_narrow_g<T, In, 8>(a, nvec, ns, s);
    case 16: return launch_n_narrow_g<T, In, 16>(a, nvec, ns, s);
    default: return launch_n_narrow_g<T, In, 32>(a, nvec, ns, s);
  }
}

// Column chunks of the wide-row F kernel: with fewer waves (frequencies x
// row groups) than half the resident wave slots, each wave would stream
// whole rows alone (few frequencies, few rows, long rows). The rows are
// then cut into ncc chunks (at most slots / waves, each at least
// kMinChunkVecsN vectors and a multiple of one step of the wave loop, so
// every load stays a contiguous 1 KiB); each wave stores its chunk's sums
// in the plan workspace and a second kernel adds the chunks in order.
constexpr int64_t kMinChunkVecsN = kWave * kUnrollN * 8;

struct ColN {
  int64_t ncc = 1, cc_len = 0;
};

int64_t resident_n_waves() { return static_cast<int64_t>(resident_c_workgroups()) / kResidentPerCuC * 4 * kWavesN; }

ColN col_n(int64_t K, int64_t Nd, int64_t nvec, int64_t wave_slots) {
  ColN cn;
  cn.cc_len = nvec;
  const int64_t waves = K * ((Nd + kRowsN - 1) / kRowsN);
  int64_t n = wave_slots / waves;
  const int64_t by_len = nvec / kMinChunkVecsN;
  n = n < by_len ? n : by_len;
  if (n < 2) return cn;
  constexpr int64_t step = kWave * kUnrollN;
  cn.cc_len = ((nvec + n - 1) / n + step - 1) / step * step;
  cn.ncc = (nvec + cn.cc_len - 1) / cn.cc_len;
  if (cn.ncc < 2) {
    cn.ncc = 1;
    cn.cc_len = nvec;
  }
  return cn;
}

size_t col_part_bytes(int64_t K, int64_t Nd, const ColN &cn) {
  return cn.ncc > 1 ? static_cast<size_t>(K * cn.ncc * Nd) * 16 : 0;  // one complex (<= 16 bytes) per row and chunk
}

// Rows of at most kShortRowVecs vectors (above the narrow form's range): a
// wave of the four-row layout finishes its rows in one or two steps and
// pays its setup and reductions for little data, so waves take kShortRows
// rows with one vector of each in flight and a single chain per row.
// Measured (mixed, Nt = 1000): Nm = 100, Nd = 5000 855 -> 672 us; Nm = 120,
// Nd = 4000 705 -> 601 us; Nm = 80, Nd = 5000 822 -> 575 us; with rows of
// 150 or 250 vectors it is slower (799 against 717 us, 651 against 604).
constexpr int64_t kShortRowVecs = 128;
constexpr int kShortRows = 16;

template <typename T, typename In>
hipError_t launch_n_wide(const SbgemvArgs &a, int64_t nvec, const ColN &cn, hipStream_t s) {
  using V = typename Vec16<T>::type;
  const int nv = Vec16<T>::n;
  cx<T> *part = static_cast<cx<T> *>(a.part);
  if (nvec <= kShortRowVecs && cn.ncc == 1) {
    const int64_t ngroups = (a.Nd + kShortRows - 1) / kShortRows;
    const int64_t ntasks = a.K * ngroups;
    const int64_t nblocks = (ntasks + (kBlock / kWave) - 1) / (kBlock / kWave);
    if (!grid_fits(nblocks, kBlock)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((sbgemv_n_kernel<T, In, kShortRows, 1, 1, kWavesN>), dim3(static_cast<unsigned>(nblocks)),
                       dim3(kBlock), 0, s, static_cast<const V *>(a.F), static_cast<const cx<In> *>(a.x), a.y, a.Nd,
                       a.ldF / nv, nvec, a.ldx, a.ldy, a.y_f32, ngroups, ntasks, nblocks, part, int64_t(1), nvec);
    return hipSuccess;
  }
  const int64_t ngroups = (a.Nd + kRowsN - 1) / kRowsN;
  const int64_t ntasks = a.K * ngroups * cn.ncc;
  const int64_t nblocks = (ntasks + (kBlock / kWave) - 1) / (kBlock / kWave);
  const int64_t nred = (a.K * a.Nd + kBlock - 1) / kBlock;
  if (!grid_fits(nblocks, kBlock) || !grid_fits(nred, kBlock)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((sbgemv_n_kernel<T, In, kRowsN, kUnrollN, kChainsN, kWavesN>), dim3(static_cast<unsigned>(nblocks)),
                     dim3(kBlock), 0, s, static_cast<const V *>(a.F), static_cast<const cx<In> *>(a.x), a.y, a.Nd,
                     a.ldF / nv, nvec, a.ldx, a.ldy, a.y_f32, ngroups, ntasks, nblocks, part, cn.ncc, cn.cc_len);
  if (cn.ncc > 1) {
    hipLaunchKernelGGL((sbgemv_n_reduce_kernel<T>), dim3(static_cast<unsigned>(nred)), dim3(kBlock), 0, s, part, a.y,
                       a.K, a.Nd, cn.ncc, a.ldy, a.y_f32);
  }
  return hipSuccess;
}

// The whole-row form of F (FP32 GEMVs): the workgroup sizes and vectors per
// lane of the conjugate-transpose whole-row form (kRowFormsC), the one that
// fills its rounds best, used only when that fill is at least kRowMinFillN
// (with fewer frequencies the four-rows-per-wave kernel, whose many short
// tasks fill any grid, stays) and the row partials fit the LDS: 64 KiB per
// workgroup, and 160 KiB per CU for all its resident workgroups (32 waves x
// 8 bytes per row: Nd <= 640), so that the slots counted are real.
// Measured on one box against the four-rows-per-wave kernel: Main (2500
// vectors, 512 x 5) 592.5 -> 588.4 us (1024 x 3: 586.7); Nm = 10000 (1024 x 5)
// 1147 -> 1140 us; the Scale share (1024 x 10) 4610 -> 4548 us; reading two
// rows per step, or 768-thread workgroups, measured slower.
constexpr double kRowMinFillN = 0.9;
constexpr int64_t kRowLdsN = 65536, kRowLdsCuN = 163840;

struct RowN {
  int tpb = 0;  // 0: not the whole-row form
  int64_t vl = 0;
};

RowN row_n(int64_t K, int64_t Nd, int64_t nvec, int64_t slots) {
  RowN best;
  if (nvec <= int64_t(kBlock) * kMaxVecsC) return best;
  double best_fill = -1.0, best_busy = 0.0;
  for (const RowFormC &f : kRowFormsC) {
    const int64_t vl = (nvec + f.tpb - 1) / f.tpb;
    if (vl < f.vl_min || vl > f.vl_max32) continue;
    const int64_t per_wg = Nd * (f.tpb / kWave) * 8;
    if (per_wg > kRowLdsN || per_wg * (int64_t(kResidentPerCuC) * kBlock / f.tpb) > kRowLdsCuN) continue;
    const int64_t s2 = slots_for(slots, f.tpb);
    const int64_t rounds = (K + s2 - 1) / s2;
    const double fill = static_cast<double>(K) / static_cast<double>(rounds * s2);
    const double busy = static_cast<double>(nvec) / static_cast<double>(vl * f.tpb);
    if (fill > best_fill + 1e-9 || (fill > best_fill - 1e-9 && busy > best_busy)) {
      best = {f.tpb, vl};
      best_fill = fill;
      best_busy = busy;
    }
  }
  if (best_fill < kRowMinFillN) best = RowN{};
  return best;
}

template <typename In, int TPB, int VL, int VLMAX>
hipError_t launch_n_row_vl(const SbgemvArgs &a, int64_t nvec, const RowN &rn, hipStream_t s) {
  if constexpr (VL > VLMAX) {
    return hipErrorInvalidValue;  // not reached: row_n keeps vl within the form's range
  } else {
    if (rn.vl != VL) return launch_n_row_vl<In, TPB, VL + 1, VLMAX>(a, nvec, rn, s);
    if (!grid_fits(a.K, TPB)) return hipErrorInvalidConfiguration;
    const size_t lds = static_cast<size_t>(a.Nd) * (TPB / kWave) * sizeof(cx<float>);
    hipLaunchKernelGGL((sbgemv_n_row_kernel<In, TPB, VL>), dim3(static_cast<unsigned>(a.K)), dim3(TPB), lds, s,
                       static_cast<const f32x4 *>(a.F), static_cast<const cx<In> *>(a.x), a.y, a.Nd, a.ldF / 2, nvec,
                       a.ldx, a.ldy, a.y_f32, a.K);
    return hipSuccess;
  }
}

template <typename In>
hipError_t launch_n_row(const SbgemvArgs &a, int64_t nvec, const RowN &rn, hipStream_t s) {
  switch (rn.tpb) {
    case 1024: return launch_n_row_vl<In, 1024, 3, 10>(a, nvec, rn, s);
    case 512: return launch_n_row_vl<In, 512, 3, 5>(a, nvec, rn, s);
    default: return launch_n_row_vl<In, 384, 4, 7>(a, nvec, rn, s);
  }
}

}  // namespace

// An FP32 GEMV reads its input vector in FP32: the buffer between stages 2
// and 3 holds the narrower precision of the two, so it is complex64 whenever
// stage 3 is FP32. The FP32 kernels read 16-byte vectors of two complex64
// entries; complex128 input there would be misread, so it is rejected.
hipError_t launch_sbgemv_n(const SbgemvArgs &a, bool compute_f32, hipStream_t s) {
  if (compute_f32 && !a.x_f32) return hipErrorInvalidValue;
  const int nv = compute_f32 ? 2 : 1;
  const int64_t nvec = (a.Nm + nv - 1) / nv;
  const NarrowSplit ns = narrow_split(a.K, a.Nd, nvec);
  hipError_t e;
  if (compute_f32) {
    const RowN rn = row_n(a.K, a.Nd, nvec, resident_c_workgroups());
    if (rn.tpb) {
      e = launch_n_row<float>(a, nvec, rn, s);
      return e != hipSuccess ? e : hipGetLastError();
    }
  }
  if (ns.G) {
    if (compute_f32)
      e = launch_n_narrow<float, float>(a, nvec, ns, s);
    else if (a.x_f32)
      e = launch_n_narrow<double, float>(a, nvec, ns, s);
    else
      e = launch_n_narrow<double, double>(a, nvec, ns, s);
    return e != hipSuccess ? e : hipGetLastError();
  }
  ColN cn = col_n(a.K, a.Nd, nvec, resident_n_waves());
  if (cn.ncc > 1 && !(a.part && a.part_bytes >= col_part_bytes(a.K, a.Nd, cn))) {
    cn.ncc = 1;  // no workspace (callers outside an apply): whole rows
    cn.cc_len = nvec;
  }
  if (compute_f32)
    e = launch_n_wide<float, float>(a, nvec, cn, s);
  else if (a.x_f32)
    e = launch_n_wide<double, float>(a, nvec, cn, s);
  else
    e = launch_n_wide<double, double>(a, nvec, cn, s);
  return e != hipSuccess ? e : hipGetLastError();
}

hipError_t launch_sbgemv_c(const SbgemvArgs &a, bool compute_f32, hipStream_t s) {
  if (compute_f32 && !a.x_f32) return hipErrorInvalidValue;  // as for launch_sbgemv_n
  const int nv = compute_f32 ? 2 : 1;
  const int64_t nvec = (a.Nm + nv - 1) / nv;
  const TallSplit ts = tall_split(a.K, a.Nd, nvec);
  const size_t need = ts.nseg ? tall_part_bytes(a.K, nvec, ts) : 0;
  hipError_t e;
  if (need && a.part && a.part_bytes >= need) {
    if (compute_f32)
      e = launch_c_tall<float, float>(a, nvec, ts, s);
    else if (a.x_f32)
      e = launch_c_tall<double, float>(a, nvec, ts, s);
    else
      e = launch_c_tall<double, double>(a, nvec, ts, s);
    return e != hipSuccess ? e : hipGetLastError();
  }
  if (compute_f32)
    e = launch_c_vl<float, float>(a, nvec, s);
  else if (a.x_f32)
    e = launch_c_vl<double, float>(a, nvec, s);
  else
    e = launch_c_vl<double, double>(a, nvec, s);
  return e != hipSuccess ? e : hipGetLastError();
}

size_t sbgemv_part_bytes(int64_t K, int64_t Nd, int64_t Nm) {
  const int64_t slots = resident_c_workgroups();
  size_t bytes = 0;
  for (int nv = 1; nv <= 2; ++nv) {
    const int64_t nvec = (Nm + nv - 1) / nv;
    if (!narrow_split(K, Nd, nvec).G) {
      const size_t bn = col_part_bytes(K, Nd, col_n(K, Nd, nvec, resident_n_waves()));
      bytes = bn > bytes ? bn : bytes;
    }
    const TallSplit ts = tall_split(K, Nd, nvec);
    size_t b = 0;
    if (ts.nseg) {
      b = tall_part_bytes(K, nvec, ts);
    } else {
      const ChunksC c = choose_chunks_c(K, nvec, slots, nv == 2);
      b = seg_part_bytes(K, nvec, seg_c(K, c, Nd, slots));
    }
    bytes = b > bytes ? b : bytes;
  }
  return bytes;
}

}  // namespace fftmv
