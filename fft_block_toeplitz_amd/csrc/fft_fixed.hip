// Batched real FFTs specialised for one transform length (stages 2 and 4
// of "Mixed-precision FFTMatvec performance optimization on AMD GPUs",
// section 1.1, for the configured workloads Nt = 1000 and Nt = 2000). Same
// algorithm as the generic kernels in fft.hip; here the schedule, butterfly
// counts and divisors are compile-time constants.
#include "fft_device.hpp"

namespace fftmv {
namespace {

// ===================================================================
// Kernels specialised for one transform length L (and C channels per
// workgroup). The schedule, the butterfly counts, every divisor and the
// zero half of the padded input are compile-time constants: no runtime
// radix dispatch (so registers are sized for this schedule only), exact
// loop trip counts, and the first forward pass never touches the inputs
// that are known to be zero. The LDS tile gets one padding row every 8 rows,
// which breaks the power-of-two strides of the early Stockham passes (bank
// conflicts).
// ===================================================================
constexpr int ct_row(int n) { return n + (n >> 3); }

// spectrum stores: non-temporal (streamed past the caches) or plain
template <bool NTS>
__device__ __forceinline__ void store_one(cx<float> *p, cx<float> v) {
  if constexpr (NTS) store_stream(p, v);
  else *p = v;
}
template <bool NTS>
__device__ __forceinline__ void store_one(cx<double> *p, cx<double> v) {
  if constexpr (NTS) store_stream(p, v);
  else *p = v;
}
template <bool NTS>
__device__ __forceinline__ void store_pair(cx<float> *p, cx<float> v0, cx<float> v1) {
  if constexpr (NTS) {
    store_stream2(p, v0, v1);
  } else {
    p[0] = v0;
    p[1] = v1;
  }
}
constexpr int ct_rows(int L) { return ct_row(L - 1) + 1; }

template <int C>
__device__ __forceinline__ int ct_idx(int n, int c) {
  return ct_row(n) * C + c;
}

template <typename T, int L, int C, int TPB, int P, int S>
__device__ __forceinline__ void ct_lds_pass(cx<T> *lds, const cx<T> *__restrict__ tw) {
  constexpr FftGeom g = make_geometry(L);
  constexpr int R = g.radix[P], NS = g.ns[P], TWS = g.twstep[P];
  constexpr int Lr = L / R, NB = Lr * C, B = (NB + TPB - 1) / TPB;
  cx<T> v[B][R];
#pragma unroll
  for (int i = 0; i < B; ++i) {
    const int b = threadIdx.x + i * TPB;
    if (NB % TPB == 0 || b < NB) {
      const int c = b % C, j = b / C;
#pragma unroll
      for (int q = 0; q < R; ++q) v[i][q] = lds[ct_idx<C>(j + q * Lr, c)];
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < B; ++i) {
    const int b = threadIdx.x + i * TPB;
    if (NB % TPB == 0 || b < NB) {
      const int c = b % C, j = b / C;
      const int k = j % NS;
      if constexpr (NS > 1) twiddle<T, R, S>(v[i], k, TWS, tw);
      dft<R, S>(v[i]);
      const int base = (j - k) * R + k;
#pragma unroll
      for (int q = 0; q < R; ++q) lds[ct_idx<C>(base + q * NS, c)] = v[i][q];
    }
  }
  __syncthreads();
}

template <typename T, int L, int C, int TPB, int P, int PEND, int S>
__device__ __forceinline__ void ct_passes(cx<T> *lds, const cx<T> *__restrict__ tw) {
  if constexpr (P < PEND) {
    ct_lds_pass<T, L, C, TPB, P, S>(lds, tw);
    ct_passes<T, L, C, TPB, P + 1, PEND, S>(lds, tw);
  }
}

// First pass (Ns = 1): inputs from get(n); inputs n >= NZ are known zeros.
template <typename T, int L, int C, int TPB, int S, int NZ, typename Get, typename Put>
__device__ __forceinline__ void ct_first_pass(Get get, Put put) {
  constexpr FftGeom g = make_geometry(L);
  constexpr int R = g.radix[0];
  constexpr int Lr = L / R, NB = Lr * C, B = (NB + TPB - 1) / TPB;
  cx<T> v[B][R];
#pragma unroll
  for (int i = 0; i < B; ++i) {
    const int b = threadIdx.x + i * TPB;
    if (NB % TPB == 0 || b < NB) {
      const int j = b / C;
#pragma unroll
      for (int q = 0; q < R; ++q) {
        if constexpr (true) {
          if (q * Lr >= NZ) {
            v[i][q] = mk(T(0), T(0));  // whole slice in the zero half
          } else if ((q + 1) * Lr <= NZ) {
            v[i][q] = get(j + q * Lr);
          } else {
            v[i][q] = j + q * Lr < NZ ? get(j + q * Lr) : mk(T(0), T(0));
          }
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < B; ++i) {
    const int b = threadIdx.x + i * TPB;
    if (NB % TPB == 0 || b < NB) {
      const int j = b / C;
      dft<R, S>(v[i]);
#pragma unroll
      for (int q = 0; q < R; ++q) put(j * R + q, v[i][q]);
    }
  }
}

// Last pass (Ns = L/R) from the LDS tile to put(n, value).
template <typename T, int L, int C, int TPB, int S, typename Put>
__device__ __forceinline__ void ct_last_pass(const cx<T> *lds, const cx<T> *__restrict__ tw, Put put) {
  constexpr FftGeom g = make_geometry(L);
  constexpr int P = g.npass - 1;
  constexpr int R = g.radix[P], TWS = g.twstep[P];
  constexpr int Lr = L / R, NB = Lr * C, B = (NB + TPB - 1) / TPB;
  cx<T> v[B][R];
#pragma unroll
  for (int i = 0; i < B; ++i) {
    const int b = threadIdx.x + i * TPB;
    if (NB % TPB == 0 || b < NB) {
      const int c = b % C, j = b / C;
#pragma unroll
      for (int q = 0; q < R; ++q) v[i][q] = lds[ct_idx<C>(j + q * Lr, c)];
    }
  }
#pragma unroll
  for (int i = 0; i < B; ++i) {
    const int b = threadIdx.x + i * TPB;
    if (NB % TPB == 0 || b < NB) {
      const int j = b / C;
      if constexpr (Lr > 1) twiddle<T, R, S>(v[i], j, TWS, tw);
      dft<R, S>(v[i]);
#pragma unroll
      for (int q = 0; q < R; ++q) put(j + q * Lr, v[i][q]);
    }
  }
}

// Forward transform of FP64 input, length L = Nt, into complex64 and/or
// complex128.
// ROUND: an FP64 transform of samples first rounded to binary32 (an FP32
// stage 1 ahead of an FP64 stage 2); FP32 transforms round on conversion.
// SETUP = false: the apply path -- one output row per frequency, 32-bit
// offsets. SETUP = true: the frequency blocks -- channel ch goes to row
// ch / cpr, column ch % cpr of its frequency's block, 64-bit offsets.
// Src: the sample type (double; float for the stage-1 buffer of the
// five-kernel form when stage 1 or 2 is FP32).
template <typename T, int L, int C, int TPB, bool NTS, bool ROUND, bool SETUP = false, typename Src = double>
__global__ __launch_bounds__(TPB) void rfft_forward_ct(FwdFftArgs a, const cx<T> *__restrict__ tw,
                                                       int64_t nblocks) {
  constexpr FftGeom g = make_geometry(L);
  static_assert(g.L == L && g.npass >= 2, "specialised kernels need at least two passes");
  __shared__ cx<T> lds[ct_rows(L) * C];
  const int c = threadIdx.x % C;
  const int64_t tile = xcd_contiguous_block(blockIdx.x, nblocks);
  const int64_t ch = tile * C + c;
  const bool live = ch < a.nchan;
  const Src *src = static_cast<const Src *>(a.src);
  const int64_t ld = a.src_ld;
  auto get = [&](int n) {
    const int t0 = 2 * n;  // t0 < L = Nt is guaranteed for n < NZ, L even or odd
    T re = T(0), im = T(0);
    if (live) {
      double x0 = static_cast<double>(load_elem<!SETUP>(src, t0 * ld + ch)), x1 = 0.0;
      if (t0 + 1 < L) x1 = static_cast<double>(load_elem<!SETUP>(src, (t0 + 1) * ld + ch));
      if constexpr (ROUND) {
        x0 = round_f32(x0);
        x1 = round_f32(x1);
      }
      re = static_cast<T>(x0);
      im = static_cast<T>(x1);
    }
    return mk(re, im);
  };
  auto to_lds = [&](int n, cx<T> v) { lds[ct_idx<C>(n, c)] = v; };
  ct_first_pass<T, L, C, TPB, -1, (L + 1) / 2>(get, to_lds);
  __syncthreads();
  ct_passes<T, L, C, TPB, 1, g.npass, -1>(lds, tw);

  // split into the Nt + 1 bins; two adjacent channels per thread so that the
  // complex64 spectrum leaves as 16-byte non-temporal stores
  constexpr int NC = C > 1 ? 2 : 1;
  constexpr int CP = C / NC;
  const int c0 = (threadIdx.x % CP) * NC;
  const int64_t ch0 = tile * C + c0;
  if (ch0 >= a.nchan) return;
  // output position of channel ch0 (and ch0 + 1 right after it when both
  // are in one row)
  int64_t o32 = ch0, o64 = ch0;
  bool two = NC == 2 && ch0 + 1 < a.nchan;
  if constexpr (SETUP) {
    const int64_t row = ch0 / a.cpr, col = ch0 - row * a.cpr;
    o32 = row * a.ldr32 + col;
    o64 = row * a.ldr64 + col;
    // a 16-byte pair store needs both channels in one row and an even
    // complex64 position (rows of odd length put odd channels at odd ones)
    two = two && col + 1 < a.cpr && (o32 & 1) == 0;
  }
  cx<float> *d32 = static_cast<cx<float> *>(a.dst32);
  cx<double> *d64 = static_cast<cx<double> *>(a.dst64);
  int64_t o32b = o32 + 1, o64b = o64 + 1;  // the second channel's position
  if constexpr (SETUP) {
    if (NC == 2 && ch0 + 1 < a.nchan) {  // ch0 + 1 may start the next row
      const int64_t row = (ch0 + 1) / a.cpr, col = ch0 + 1 - row * a.cpr;
      o32b = row * a.ldr32 + col;
      o64b = row * a.ldr64 + col;
    }
  }
  const bool second = NC == 2 && ch0 + 1 < a.nchan;
  for (int b = threadIdx.x; b < (L + 1) * CP; b += TPB) {
    const int k = b / CP;
    const int ka = k == L ? 0 : k, kb = k == 0 ? 0 : L - k;
    const cx<T> w = tw[k];
    cx<T> x[NC];
#pragma unroll
    for (int e = 0; e < NC; ++e) {
      cx<T> za = lds[ct_idx<C>(ka, c0 + e)], zb = conj(lds[ct_idx<C>(kb, c0 + e)]);
      cx<T> ev = scale(za + zb, T(0.5));
      cx<T> dd = za - zb;
      x[e] = ev + cmul(mk(dd.im * T(0.5), -dd.re * T(0.5)), w);
    }
    if (d32) {
      cx<float> *p = d32 + k * a.fstride32;
      if (two) {
        store_pair<NTS>(p + o32, cvt<float>(x[0]), cvt<float>(x[NC - 1]));
      } else {
        store_one<NTS>(p + o32, cvt<float>(x[0]));
        if (second) store_one<NTS>(p + o32b, cvt<float>(x[NC - 1]));
      }
    }
    if (d64) {
      cx<double> *p = d64 + k * a.fstride64;
      store_one<NTS>(p + o64, cvt<double>(x[0]));
      if (second) store_one<NTS>(p + o64b, cvt<double>(x[NC - 1]));
    }
  }
}

template <typename T, typename Src, int L, int C, int TPB>
__global__ __launch_bounds__(TPB) void rfft_inverse_ct(InvFftArgs a, const cx<T> *__restrict__ tw, T inv_l,
                                                          int64_t nblocks) {
  constexpr FftGeom g = make_geometry(L);
  static_assert(g.L == L && g.npass >= 2, "specialised kernels need at least two passes");
  __shared__ cx<T> lds[ct_rows(L) * C];
  const int c = threadIdx.x % C;
  const int64_t ch = xcd_contiguous_block(blockIdx.x, nblocks) * C + c;
  const bool live = ch < a.nchan;
  const cx<Src> *src = static_cast<const cx<Src> *>(a.src);
  const int64_t ld = a.src_ld, dld = a.dst_ld;
  auto get = [&](int k) {
    if (!live) return mk(T(0), T(0));
    cx<T> xa = cvt<T>(load_elem<true>(src, k * ld + ch));
    cx<T> xb = cvt<T>(load_elem<true>(src, (L - k) * ld + ch));
    if (k == 0) {
      xa.im = T(0);
      xb.im = T(0);
    }
    xb = conj(xb);
    cx<T> e = scale(xa + xb, T(0.5));
    cx<T> o = scale(cmulc(xa - xb, tw[k]), T(0.5));
    return mk(e.re - o.im, e.im + o.re);
  };
  auto put = [&](int n, cx<T> z) {
    const int t0 = 2 * n;
    if (!live || t0 >= L) return;
    const bool second = t0 + 1 < L;
    const T y0 = z.re * inv_l, y1 = z.im * inv_l;
    if (a.dst_f32) {
      float *d = static_cast<float *>(a.dst);
      store_elem<true>(d, t0 * dld + ch, static_cast<float>(y0));
      if (second) store_elem<true>(d, (t0 + 1) * dld + ch, static_cast<float>(y1));
    } else {
      double *d = static_cast<double *>(a.dst);
      double v0 = static_cast<double>(y0), v1 = static_cast<double>(y1);
      if (a.round_f32) {
        v0 = round_f32(v0);
        v1 = round_f32(v1);
      }
      store_elem<true>(d, t0 * dld + ch, v0);
      if (second) store_elem<true>(d, (t0 + 1) * dld + ch, v1);
    }
  };
  auto to_lds = [&](int n, cx<T> v) { lds[ct_idx<C>(n, c)] = v; };
  ct_first_pass<T, L, C, TPB, +1, L>(get, to_lds);
  __syncthreads();
  ct_passes<T, L, C, TPB, 1, g.npass - 1, +1>(lds, tw);
  ct_last_pass<T, L, C, TPB, +1>(lds, tw, put);
}

// Lengths with specialised kernels (the configured workloads: Nt = 1000 and
// Nt = 2000) and the tile for wide batches: C channels per workgroup so that
// each frequency row of the output is written in 64-byte runs, with enough
// threads for the C*L/R butterflies of a pass. Measured at Nt = 1000,
// FP32, 5000 channels: 8 channels x 512 threads beat 4 x 256 (forward
// 25 us vs 47 us; the 32-byte runs of the narrower tile double the bytes
// the non-temporal stores write), 16 x 1024 and 10 unpadded x 640 (which
// fits the batch in one round but loses more to its 80-byte runs); 8 x 1024
// (one butterfly per thread and pass, two workgroups per CU) saves another
// ~2 us per transform over 8 x 512.
struct CtTile {
  int C, tpb;
};
template <typename T>
constexpr CtTile ct_wide_tile(int L) {
  return L == 1000 ? CtTile{sizeof(T) == 4 ? 8 : 4, sizeof(T) == 4 ? 1024 : 512}
                   : CtTile{sizeof(T) == 4 ? 8 : 4, 1024};
}
constexpr bool has_ct(int L) { return L == 1000 || L == 2000; }
constexpr int64_t kWideBatch = 4096;  // channels from which wide tiles pay

template <typename T, int L, bool ROUND, typename Src, int C, int TPB = kBlock>
void launch_fwd_ct(const FwdFftArgs &a, const void *tw, hipStream_t s) {
  const int64_t nblocks = (a.nchan + C - 1) / C;
  hipLaunchKernelGGL((rfft_forward_ct<T, L, C, TPB, true, ROUND, false, Src>), dim3(static_cast<unsigned>(nblocks)),
                     dim3(TPB), 0, s, a, static_cast<const cx<T> *>(tw), nblocks);
}

template <typename T, int L, bool ROUND, typename Src = double>
void launch_fwd_ct_c(const FwdFftArgs &a, const void *tw, hipStream_t s) {
  constexpr CtTile w = ct_wide_tile<T>(L);
  if (a.nchan >= kWideBatch)
    launch_fwd_ct<T, L, ROUND, Src, w.C, w.tpb>(a, tw, s);
  else
    launch_fwd_ct<T, L, ROUND, Src, 1>(a, tw, s);
}

// the frequency blocks (setup): FP64 transform, 64-bit offsets, rows of cpr
// channels. Plain (cached) stores: nothing follows in the same stream that
// the written lines could slow down, and partial lines of neighbouring
// tiles merge in L2 instead of reaching HBM twice. At Nt = 1000 the tile
// holds 8 channels (144 KB of LDS), so every time step of F is read in
// 64-byte runs; at Nt = 2000 four channels already fill the LDS.
template <int L>
void launch_fwd_ct_setup(const FwdFftArgs &a, const void *tw, hipStream_t s) {
  constexpr int C = L == 1000 ? 8 : 4, TPB = 1024;
  const cx<double> *t = static_cast<const cx<double> *>(tw);
  if (a.nchan >= kWideBatch) {
    const int64_t nblocks = (a.nchan + C - 1) / C;
    hipLaunchKernelGGL((rfft_forward_ct<double, L, C, TPB, false, false, true>), dim3(static_cast<unsigned>(nblocks)),
                       dim3(TPB), 0, s, a, t, nblocks);
  } else {
    hipLaunchKernelGGL((rfft_forward_ct<double, L, 1, kBlock, false, false, true>),
                       dim3(static_cast<unsigned>(a.nchan)), dim3(kBlock), 0, s, a, t, a.nchan);
  }
}

template <int L>
void launch_fwd_ct_any(const FwdFftArgs &a, bool compute_f32, const void *tw, hipStream_t s) {
  if (a.src_f32) {  // the stage-1 buffer of the five-kernel form (already rounded)
    if (compute_f32)
      launch_fwd_ct_c<float, L, false, float>(a, tw, s);
    else
      launch_fwd_ct_c<double, L, false, float>(a, tw, s);
    return;
  }
  if (compute_f32)
    launch_fwd_ct_c<float, L, false>(a, tw, s);  // conversion to float rounds
  else if (a.round_f32)
    launch_fwd_ct_c<double, L, true>(a, tw, s);
  else
    launch_fwd_ct_c<double, L, false>(a, tw, s);
}

// the specialised forward kernel covers the apply path: FP64 input, one
// output row per frequency, byte offsets below 4 GiB
bool fwd_ct_applies(const FftGeom &g, const FwdFftArgs &a) {
  return has_ct(g.L) && a.Nt == g.L && !(a.src_f32 && a.round_f32) && a.cpr >= a.nchan &&
         fits_32bit(a.Nt, a.src_ld, 8) && a.nchan <= a.src_ld;
}

template <typename T, typename Src, int L, int C, int TPB = kBlock>
void launch_inv_ct(const InvFftArgs &a, const void *tw, hipStream_t s) {
  const int64_t nblocks = (a.nchan + C - 1) / C;
  hipLaunchKernelGGL((rfft_inverse_ct<T, Src, L, C, TPB>), dim3(static_cast<unsigned>(nblocks)), dim3(TPB), 0, s,
                     a, static_cast<const cx<T> *>(tw), T(1) / static_cast<T>(L), nblocks);
}

template <typename T, typename Src, int L>
void launch_inv_ct_c(const InvFftArgs &a, const void *tw, hipStream_t s) {
  constexpr CtTile w = ct_wide_tile<T>(L);
  if (a.nchan >= kWideBatch)
    launch_inv_ct<T, Src, L, w.C, w.tpb>(a, tw, s);
  else
    launch_inv_ct<T, Src, L, 1>(a, tw, s);
}

template <typename T, typename Src>
void launch_inv_ct_any(const FftGeom &g, const InvFftArgs &a, const void *tw, hipStream_t s) {
  if (g.L == 1000)
    launch_inv_ct_c<T, Src, 1000>(a, tw, s);
  else
    launch_inv_ct_c<T, Src, 2000>(a, tw, s);
}

bool inv_ct_applies(const FftGeom &g, const InvFftArgs &a) {
  return has_ct(g.L) && a.Nt == g.L && fits_32bit(g.L + 1, a.src_ld, a.src_f32 ? 8 : 16) &&
         fits_32bit(a.Nt, a.dst_ld, 8) && a.nchan <= a.src_ld && a.nchan <= a.dst_ld;
}


}  // namespace

bool launch_fft_forward_fixed(const FftGeom &g, const FwdFftArgs &a, bool compute_f32, const void *tw,
                              hipStream_t s) {
  if (!fwd_ct_applies(g, a)) {
    // the frequency blocks: FP64 input and transform, any row structure and size
    const bool setup = has_ct(g.L) && a.Nt == g.L && !a.src_f32 && !a.round_f32 && !compute_f32 &&
                       a.nchan <= a.src_ld && a.cpr >= 1 && (a.nchan + kWideBatch) / 4 < INT32_MAX;
    if (!setup) return false;
    if (g.L == 1000)
      launch_fwd_ct_setup<1000>(a, tw, s);
    else
      launch_fwd_ct_setup<2000>(a, tw, s);
    return true;
  }
  if (g.L == 1000)
    launch_fwd_ct_any<1000>(a, compute_f32, tw, s);
  else
    launch_fwd_ct_any<2000>(a, compute_f32, tw, s);
  return true;
}

bool launch_fft_inverse_fixed(const FftGeom &g, const InvFftArgs &a, bool compute_f32, const void *tw,
                              hipStream_t s) {
  if (!inv_ct_applies(g, a)) return false;
  if (compute_f32 && a.src_f32) launch_inv_ct_any<float, float>(g, a, tw, s);
  else if (compute_f32) launch_inv_ct_any<float, double>(g, a, tw, s);
  else if (a.src_f32) launch_inv_ct_any<double, float>(g, a, tw, s);
  else launch_inv_ct_any<double, double>(g, a, tw, s);
  return true;
}

}  // namespace fftmv
