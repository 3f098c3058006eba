// Batched real FFTs along time for the block-Toeplitz matvec: stage 2
// (forward, time -> frequency) and stage 4 (inverse, frequency -> time) of
// "Mixed-precision FFTMatvec performance optimization on AMD GPUs",
// section 1.1. The same forward kernel builds the frequency blocks at setup.
//
// A length N = 2L real transform is carried by one length-L complex
// transform of z[n] = x[2n] + i x[2n+1] (even samples in the real part, odd
// samples in the imaginary part), split afterwards with
//   X[k] = E[k] + w^k O[k],  E = (Z[k] + conj Z[L-k]) / 2,
//                            O = (Z[k] - conj Z[L-k]) / 2i,  w = exp(-2 pi i / N)
// and run backwards for the inverse. The zero half of the padded input
// (section 1.1, stage 1) is never loaded: samples at t >= Nt are zeros by
// construction; the inverse only produces the Nt samples the unpad keeps.
//
// One workgroup transforms C channels at once (C a power of two). The data
// sit in LDS as [L][C] complex, channel fastest, so consecutive lanes touch
// consecutive channels: global loads and stores along a time step or a
// frequency are contiguous over the C channels, and LDS accesses are
// stride-1 across lanes. The length-L complex FFT is a Stockham autosort
// (self-sorting, no bit reversal) with radix 2/3/4/5/7/8 passes; each pass reads
// all its butterfly inputs into registers, synchronises, then writes in
// place. The first pass takes its inputs straight from global memory (all
// of a thread's loads in flight at once) and, in the inverse, the last pass
// stores straight to global memory, so the data cross LDS only between
// passes. Channel tiles are numbered XCD-contiguously so that neighbouring
// tiles, which share cache lines, share an L2.
#pragma once

#include <atomic>
#include <cstdint>

#include "fft_device.hpp"

namespace fftmv {
namespace {

// A thread keeps at most VMAX complex values in registers during a pass,
// i.e. VMAX / R butterflies of radix R: kVmax in 256-thread workgroups,
// kVmaxWide in 1024-thread ones (which fit 128 VGPRs per lane). The host
// picks C (channels per workgroup) and the workgroup size so that every
// pass of the schedule fits; with C = 1 every supported length fits, the
// longest radix-7 schedules (Nt above 3584) in 1024-thread workgroups.
constexpr int kVmax = 20;
constexpr int kVmaxWide = 10;
// One Stockham pass of radix R over the [L][C] LDS tile. Butterfly j of
// channel c reads elements j + q L/R, multiplies input q by
// w_{Ns R}^{(j mod Ns) q} and writes output q to (j - j mod Ns) R + j mod Ns + q Ns.
template <typename T, int R, int S, int VMAX, int TPB>
__device__ __forceinline__ void lds_pass(cx<T> *lds, int L, int logC, int Ns, int twstep,
                                         const cx<T> *__restrict__ tw) {
  constexpr int B = VMAX / R;
  const int C = 1 << logC;
  const int Lr = L / R;
  const int nb = Lr << logC;
  cx<T> v[B][R];
#pragma unroll
  for (int i = 0; i < B; ++i) {
    int b = threadIdx.x + i * TPB;
    if (b < nb) {
      int c = b & (C - 1), j = b >> logC;
#pragma unroll
      for (int q = 0; q < R; ++q) v[i][q] = lds[((j + q * Lr) << logC) + c];
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < B; ++i) {
    int b = threadIdx.x + i * TPB;
    if (b < nb) {
      int c = b & (C - 1), j = b >> logC;
      int k = j % Ns;
      if (Ns > 1) twiddle<T, R, S>(v[i], k, twstep, tw);
      dft<R, S>(v[i]);
      int base = (j - k) * R + k;
#pragma unroll
      for (int q = 0; q < R; ++q) lds[((base + q * Ns) << logC) + c] = v[i][q];
    }
  }
  __syncthreads();
}

// First pass (Ns = 1, no twiddles): input n of this thread's channel comes
// from get(n), output n goes to put(n, value). All loads of the thread are
// issued before any butterfly.
template <typename T, int R, int S, int VMAX, int TPB, typename Get, typename Put>
__device__ __forceinline__ void first_pass(int L, int logC, Get get, Put put) {
  constexpr int B = VMAX / R;
  const int Lr = L / R;
  const int nb = Lr << logC;
  cx<T> v[B][R];
#pragma unroll
  for (int i = 0; i < B; ++i) {
    int b = threadIdx.x + i * TPB;
    if (b < nb) {
      int j = b >> logC;
#pragma unroll
      for (int q = 0; q < R; ++q) v[i][q] = get(j + q * Lr);
    }
  }
#pragma unroll
  for (int i = 0; i < B; ++i) {
    int b = threadIdx.x + i * TPB;
    if (b < nb) {
      int j = b >> logC;
      dft<R, S>(v[i]);
#pragma unroll
      for (int q = 0; q < R; ++q) put(j * R + q, v[i][q]);
    }
  }
}

// Last pass (Ns = L/R) reading the LDS tile and handing output n to put.
template <typename T, int R, int S, int VMAX, int TPB, typename Put>
__device__ __forceinline__ void last_pass(const cx<T> *lds, int L, int logC, int twstep,
                                          const cx<T> *__restrict__ tw, Put put) {
  constexpr int B = VMAX / R;
  const int C = 1 << logC;
  const int Lr = L / R;  // == Ns of this pass
  const int nb = Lr << logC;
  cx<T> v[B][R];
#pragma unroll
  for (int i = 0; i < B; ++i) {
    int b = threadIdx.x + i * TPB;
    if (b < nb) {
      int c = b & (C - 1), j = b >> logC;
#pragma unroll
      for (int q = 0; q < R; ++q) v[i][q] = lds[((j + q * Lr) << logC) + c];
    }
  }
#pragma unroll
  for (int i = 0; i < B; ++i) {
    int b = threadIdx.x + i * TPB;
    if (b < nb) {
      int j = b >> logC;
      if (Lr > 1) twiddle<T, R, S>(v[i], j, twstep, tw);
      dft<R, S>(v[i]);
#pragma unroll
      for (int q = 0; q < R; ++q) put(j + q * Lr, v[i][q]);
    }
  }
}

template <typename T, int S, int VMAX, int TPB>
__device__ __forceinline__ void middle_passes(cx<T> *lds, const FftGeom &g, int first, int last, int logC,
                                              const cx<T> *__restrict__ tw) {
  for (int p = first; p < last; ++p) {
    switch (g.radix[p]) {
      case 2: lds_pass<T, 2, S, VMAX, TPB>(lds, g.L, logC, g.ns[p], g.twstep[p], tw); break;
      case 3: lds_pass<T, 3, S, VMAX, TPB>(lds, g.L, logC, g.ns[p], g.twstep[p], tw); break;
      case 4: lds_pass<T, 4, S, VMAX, TPB>(lds, g.L, logC, g.ns[p], g.twstep[p], tw); break;
      case 5: lds_pass<T, 5, S, VMAX, TPB>(lds, g.L, logC, g.ns[p], g.twstep[p], tw); break;
      case 7: lds_pass<T, 7, S, VMAX, TPB>(lds, g.L, logC, g.ns[p], g.twstep[p], tw); break;
      default: lds_pass<T, 8, S, VMAX, TPB>(lds, g.L, logC, g.ns[p], g.twstep[p], tw); break;
    }
  }
}

template <typename T, int S, int VMAX, int TPB, typename Get, typename Put>
__device__ __forceinline__ void first_pass_any(int R, int L, int logC, Get get, Put put) {
  switch (R) {
    case 2: first_pass<T, 2, S, VMAX, TPB>(L, logC, get, put); break;
    case 3: first_pass<T, 3, S, VMAX, TPB>(L, logC, get, put); break;
    case 4: first_pass<T, 4, S, VMAX, TPB>(L, logC, get, put); break;
    case 5: first_pass<T, 5, S, VMAX, TPB>(L, logC, get, put); break;
    case 7: first_pass<T, 7, S, VMAX, TPB>(L, logC, get, put); break;
    default: first_pass<T, 8, S, VMAX, TPB>(L, logC, get, put); break;
  }
}

template <typename T, int S, int VMAX, int TPB, typename Put>
__device__ __forceinline__ void last_pass_any(int R, const cx<T> *lds, int L, int logC, int twstep,
                                              const cx<T> *__restrict__ tw, Put put) {
  switch (R) {
    case 2: last_pass<T, 2, S, VMAX, TPB>(lds, L, logC, twstep, tw, put); break;
    case 3: last_pass<T, 3, S, VMAX, TPB>(lds, L, logC, twstep, tw, put); break;
    case 4: last_pass<T, 4, S, VMAX, TPB>(lds, L, logC, twstep, tw, put); break;
    case 5: last_pass<T, 5, S, VMAX, TPB>(lds, L, logC, twstep, tw, put); break;
    case 7: last_pass<T, 7, S, VMAX, TPB>(lds, L, logC, twstep, tw, put); break;
    default: last_pass<T, 8, S, VMAX, TPB>(lds, L, logC, twstep, tw, put); break;
  }
}
template <typename T, typename Src, bool ROUND>
__device__ __forceinline__ T to_compute(Src v) {
  if constexpr (ROUND && sizeof(Src) == 8) return static_cast<T>(round_f32(v));
  return static_cast<T>(v);
}

// --------------------------------------------------------------- forward
// BLUE: the length-L complex FFT in Bluestein form over an M-point tile
// (g is then the schedule of M; tw stays the w_{2L} table, twM is w_{2M},
// hM the filter's transform).
template <typename T, typename Src, bool ROUND, int VMAX, bool OFF32, bool BLUE, int TPB>
__global__ __launch_bounds__(TPB) void rfft_forward_kernel(FftGeom g, FwdFftArgs a, int logC,
                                                              const cx<T> *__restrict__ tw, int64_t nblocks,
                                                              const cx<T> *__restrict__ twM,
                                                              const cx<T> *__restrict__ hM) {
  extern __shared__ __align__(16) unsigned char smem[];
  cx<T> *lds = reinterpret_cast<cx<T> *>(smem);
  const int C = 1 << logC;
  const int L = static_cast<int>(a.Nt);
  // chirp c[m] = exp(-pi i m^2 / L) (m < L <= 2048: m^2 fits 32 bits)
  auto chirp = [&](int m) { return tw[(m * m) % (2 * L)]; };
  const int c = threadIdx.x & (C - 1);  // fixed per thread: TPB is a multiple of C
  const int64_t ch = xcd_contiguous_block(blockIdx.x, nblocks) * C + c;
  const bool live = ch < a.nchan;
  const Src *src = static_cast<const Src *>(a.src);
  const int64_t Nt = a.Nt, ld = a.src_ld;

  // stages 1-2 boundary: packed samples z[n] = x[2n] + i x[2n+1]; samples at
  // t >= Nt are the zero padding and are not read
  auto get = [&](int n) {
    const int64_t t0 = 2 * static_cast<int64_t>(n);
    T re = T(0), im = T(0);
    if (live && t0 < Nt) re = to_compute<T, Src, ROUND>(load_elem<OFF32>(src, t0 * ld + ch));
    if (live && t0 + 1 < Nt) im = to_compute<T, Src, ROUND>(load_elem<OFF32>(src, (t0 + 1) * ld + ch));
    return mk(re, im);
  };
  auto to_lds = [&](int n, cx<T> v) { lds[(n << logC) + c] = v; };
  if constexpr (BLUE) {
    // a[n] = z[n] c[n], zero up to M; a * conj(c) by M-point transforms
    const int M = g.L;
    auto get_a = [&](int n) { return n < L ? cmul(get(n), chirp(n)) : mk(T(0), T(0)); };
    first_pass_any<T, -1, VMAX, TPB>(g.radix[0], M, logC, get_a, to_lds);
    __syncthreads();
    middle_passes<T, -1, VMAX, TPB>(lds, g, 1, g.npass, logC, twM);
    for (int i = threadIdx.x; i < (M << logC); i += TPB) lds[i] = cmul(lds[i], hM[i >> logC]);
    __syncthreads();
    middle_passes<T, +1, VMAX, TPB>(lds, g, 0, g.npass, logC, twM);
  } else {
    if (g.npass == 0) {  // L == 1
      if (threadIdx.x < C) to_lds(0, get(0));
    } else {
      first_pass_any<T, -1, VMAX, TPB>(g.radix[0], L, logC, get, to_lds);
    }
    __syncthreads();
    middle_passes<T, -1, VMAX, TPB>(lds, g, 1, g.npass, logC, tw);
  }
  // Z[k]: the tile entry (times c[k] in Bluestein form)
  auto zat = [&](int k, int ch) {
    cx<T> v = lds[(k << logC) + ch];
    if constexpr (BLUE) v = cmul(v, chirp(k));
    return v;
  };

  // X[k] for k = 0..L; each thread takes two adjacent channels of one bin so
  // that the complex64 output goes out as 16-byte stores
  const int half = C > 1 ? C / 2 : 1;
  const int logh = C > 1 ? logC - 1 : 0;
  const int cp = threadIdx.x & (half - 1);
  const int c0 = C > 1 ? 2 * cp : 0;
  const int nc = C > 1 ? 2 : 1;
  const int64_t ch0 = xcd_contiguous_block(blockIdx.x, nblocks) * C + c0;
  if (ch0 >= a.nchan) return;
  const bool two = nc == 2 && ch0 + 1 < a.nchan;
  const int64_t row0 = ch0 / a.cpr, col0 = ch0 - row0 * a.cpr;
  const int64_t row1 = two ? (ch0 + 1) / a.cpr : row0, col1 = two ? ch0 + 1 - row1 * a.cpr : col0;
  cx<float> *d32a = a.dst32 ? static_cast<cx<float> *>(a.dst32) + row0 * a.ldr32 + col0 : nullptr;
  cx<float> *d32b = a.dst32 ? static_cast<cx<float> *>(a.dst32) + row1 * a.ldr32 + col1 : nullptr;
  cx<double> *d64a = a.dst64 ? static_cast<cx<double> *>(a.dst64) + row0 * a.ldr64 + col0 : nullptr;
  cx<double> *d64b = a.dst64 ? static_cast<cx<double> *>(a.dst64) + row1 * a.ldr64 + col1 : nullptr;
  // one 16-byte store when both outputs are adjacent and 16-byte aligned
  // (frequency strides are even)
  const bool pack32 = two && d32b == d32a + 1 && (reinterpret_cast<uintptr_t>(d32a) & 15) == 0 &&
                      (a.fstride32 & 1) == 0;
  for (int b = threadIdx.x; b < ((L + 1) << logh); b += TPB) {
    const int k = b >> logh;
    const int ka = k == L ? 0 : k, kb = k == 0 ? 0 : L - k;
    const cx<T> w = tw[k];
    cx<T> x[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      if (e == 1 && !two) break;
      cx<T> za = zat(ka, c0 + e), zb = conj(zat(kb, c0 + e));
      cx<T> ev = scale(za + zb, T(0.5));
      cx<T> dd = za - zb;
      cx<T> o = mk(dd.im * T(0.5), -dd.re * T(0.5));  // (za - zb) / 2i
      x[e] = ev + cmul(o, w);
    }
    // non-temporal when the tile holds several channels: the spectrum is
    // consumed by the next kernel, not by this one, and streaming it out
    // keeps it from lingering dirty in the caches. One channel per
    // workgroup stores plainly: its bins share each cache line with those of
    // neighbouring workgroups, and the partial lines merge in L2.
    if (d64a) {
      if (C > 1) {
        store_stream(d64a + k * a.fstride64, cvt<double>(x[0]));
        if (two) store_stream(d64b + k * a.fstride64, cvt<double>(x[1]));
      } else {
        d64a[k * a.fstride64] = cvt<double>(x[0]);
      }
    }
    if (d32a) {
      if (pack32) {
        store_stream2(d32a + k * a.fstride32, cvt<float>(x[0]), cvt<float>(x[1]));
      } else if (C > 1) {
        store_stream(d32a + k * a.fstride32, cvt<float>(x[0]));
        if (two) store_stream(d32b + k * a.fstride32, cvt<float>(x[1]));
      } else {
        d32a[k * a.fstride32] = cvt<float>(x[0]);
      }
    }
  }
}

// --------------------------------------------------------------- inverse
template <typename T, typename Src, int VMAX, bool OFF32, bool BLUE, int TPB>
__global__ __launch_bounds__(TPB) void rfft_inverse_kernel(FftGeom g, InvFftArgs a, int logC,
                                                              const cx<T> *__restrict__ tw, T inv_l,
                                                              int64_t nblocks, const cx<T> *__restrict__ twM,
                                                              const cx<T> *__restrict__ hM) {
  extern __shared__ __align__(16) unsigned char smem[];
  cx<T> *lds = reinterpret_cast<cx<T> *>(smem);
  const int C = 1 << logC;
  const int L = static_cast<int>(a.Nt);
  auto chirp = [&](int m) { return tw[(m * m) % (2 * L)]; };
  const int c = threadIdx.x & (C - 1);
  const int64_t ch = xcd_contiguous_block(blockIdx.x, nblocks) * C + c;
  const bool live = ch < a.nchan;
  const cx<Src> *src = static_cast<const cx<Src> *>(a.src);
  const int64_t Nt = a.Nt, ld = a.src_ld, dld = a.dst_ld;

  // Z[k] = E[k] + i O[k] with E = (X[k] + conj X[L-k]) / 2 and
  // O = (X[k] - conj X[L-k]) conj(w^k) / 2; the imaginary parts of bins 0
  // and L (= Nt) are dropped, as a real signal's spectrum has none
  auto get = [&](int k) {
    if (!live) return mk(T(0), T(0));
    cx<T> xa = cvt<T>(load_elem<OFF32>(src, static_cast<int64_t>(k) * ld + ch));
    cx<T> xb = cvt<T>(load_elem<OFF32>(src, static_cast<int64_t>(L - k) * ld + ch));
    if (k == 0) {
      xa.im = T(0);
      xb.im = T(0);
    }
    xb = conj(xb);
    cx<T> e = scale(xa + xb, T(0.5));
    cx<T> o = scale(cmulc(xa - xb, tw[k]), T(0.5));
    return mk(e.re - o.im, e.im + o.re);
  };
  // stage 4-5 boundary: z[n] = y[2n] + i y[2n+1]; keep t < Nt only
  auto put = [&](int n, cx<T> z) {
    const int64_t t0 = 2 * static_cast<int64_t>(n);
    if (!live || t0 >= Nt) return;
    const bool second = t0 + 1 < Nt;
    const T y0 = z.re * inv_l, y1 = z.im * inv_l;
    if (a.dst_f32) {
      float *d = static_cast<float *>(a.dst);
      store_elem<OFF32>(d, t0 * dld + ch, static_cast<float>(y0));
      if (second) store_elem<OFF32>(d, (t0 + 1) * dld + ch, static_cast<float>(y1));
    } else {
      double *d = static_cast<double *>(a.dst);
      double v0 = static_cast<double>(y0), v1 = static_cast<double>(y1);
      if (a.round_f32) {
        v0 = round_f32(v0);
        v1 = round_f32(v1);
      }
      store_elem<OFF32>(d, t0 * dld + ch, v0);
      if (second) store_elem<OFF32>(d, (t0 + 1) * dld + ch, v1);
    }
  };
  auto to_lds = [&](int n, cx<T> v) { lds[(n << logC) + c] = v; };

  if constexpr (BLUE) {
    // a[k] = Z[k] conj(c[k]), zero up to M; a * c by M-point transforms;
    // z[n] = conj(c[n]) (a * c)[n]
    const int M = g.L;
    auto get_a = [&](int k) { return k < L ? cmulc(get(k), chirp(k)) : mk(T(0), T(0)); };
    auto put_z = [&](int n, cx<T> v) {
      if (n < L) put(n, cmulc(v, chirp(n)));
    };
    first_pass_any<T, -1, VMAX, TPB>(g.radix[0], M, logC, get_a, to_lds);
    __syncthreads();
    middle_passes<T, -1, VMAX, TPB>(lds, g, 1, g.npass, logC, twM);
    for (int i = threadIdx.x; i < (M << logC); i += TPB) lds[i] = cmul(lds[i], hM[i >> logC]);
    __syncthreads();
    middle_passes<T, +1, VMAX, TPB>(lds, g, 0, g.npass - 1, logC, twM);
    const int pl = g.npass - 1;
    last_pass_any<T, +1, VMAX, TPB>(g.radix[pl], lds, M, logC, g.twstep[pl], twM, put_z);
    return;
  }
  if (g.npass == 0) {  // L == 1
    if (threadIdx.x < C) put(0, get(0));
    return;
  }
  if (g.npass == 1) {
    first_pass_any<T, +1, VMAX, TPB>(g.radix[0], L, logC, get, put);
    return;
  }
  first_pass_any<T, +1, VMAX, TPB>(g.radix[0], L, logC, get, to_lds);
  __syncthreads();
  middle_passes<T, +1, VMAX, TPB>(lds, g, 1, g.npass - 1, logC, tw);
  const int pl = g.npass - 1;
  last_pass_any<T, +1, VMAX, TPB>(g.radix[pl], lds, L, logC, g.twstep[pl], tw, put);
}

int ilog2(int c) {
  int l = 0;
  while ((1 << l) < c) ++l;
  return l;
}

// Launch one batched transform with the generic kernels. tile: the
// schedule of the LDS tile (length L, or M in Bluestein form); twM, hM: the
// Bluestein tables (BLUE only).
// Wide workgroups may take more than 64 KiB of dynamic LDS: raise the
// kernel's limit, once per device (a function attribute is per device);
// `done` holds one bit per device already raised.
inline hipError_t raise_wide_lds(const void *kernel, std::atomic<uint64_t> &done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? uint64_t(1) << dev : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLdsWide);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}

template <typename T, typename Src, bool ROUND, bool BLUE, int TPB>
hipError_t fwd_tpb(const FftGeom &tile, const FwdFftArgs &a, const FftLaunch &cfg, const void *tw,
                   const void *twM, const void *hM, hipStream_t s) {
  const int64_t nblocks = (a.nchan + cfg.C - 1) / cfg.C;
  const size_t lds = static_cast<size_t>(tile.L) * cfg.C * sizeof(cx<T>);
  auto *k = &rfft_forward_kernel<T, Src, ROUND, TPB == kBlockWide ? kVmaxWide : kVmax, false, BLUE, TPB>;
  if constexpr (TPB == kBlockWide) {
    static std::atomic<uint64_t> raised{0};
    const hipError_t e = raise_wide_lds(reinterpret_cast<const void *>(k), raised);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(nblocks)), dim3(TPB), lds, s, tile, a, ilog2(cfg.C),
                     static_cast<const cx<T> *>(tw), nblocks, static_cast<const cx<T> *>(twM),
                     static_cast<const cx<T> *>(hM));
  return hipSuccess;
}
template <typename T, typename Src, bool ROUND, bool BLUE>
hipError_t fwd(const FftGeom &tile, const FwdFftArgs &a, const FftLaunch &cfg, const void *tw, const void *twM,
               const void *hM, hipStream_t s) {
  if (cfg.tpb == kBlockWide) return fwd_tpb<T, Src, ROUND, BLUE, kBlockWide>(tile, a, cfg, tw, twM, hM, s);
  return fwd_tpb<T, Src, ROUND, BLUE, kBlock>(tile, a, cfg, tw, twM, hM, s);
}

template <typename T, typename Src, bool BLUE, int TPB>
hipError_t inv_tpb(const FftGeom &tile, const InvFftArgs &a, const FftLaunch &cfg, const void *tw,
                   const void *twM, const void *hM, hipStream_t s) {
  const int64_t nblocks = (a.nchan + cfg.C - 1) / cfg.C;
  const size_t lds = static_cast<size_t>(tile.L) * cfg.C * sizeof(cx<T>);
  auto *k = &rfft_inverse_kernel<T, Src, TPB == kBlockWide ? kVmaxWide : kVmax, false, BLUE, TPB>;
  if constexpr (TPB == kBlockWide) {
    static std::atomic<uint64_t> raised{0};
    const hipError_t e = raise_wide_lds(reinterpret_cast<const void *>(k), raised);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(nblocks)), dim3(TPB), lds, s, tile, a, ilog2(cfg.C),
                     static_cast<const cx<T> *>(tw), T(1) / static_cast<T>(a.Nt), nblocks,
                     static_cast<const cx<T> *>(twM), static_cast<const cx<T> *>(hM));
  return hipSuccess;
}
template <typename T, typename Src, bool BLUE>
hipError_t inv(const FftGeom &tile, const InvFftArgs &a, const FftLaunch &cfg, const void *tw, const void *twM,
               const void *hM, hipStream_t s) {
  if (cfg.tpb == kBlockWide) return inv_tpb<T, Src, BLUE, kBlockWide>(tile, a, cfg, tw, twM, hM, s);
  return inv_tpb<T, Src, BLUE, kBlock>(tile, a, cfg, tw, twM, hM, s);
}

// the element types of one launch
template <bool BLUE>
hipError_t fwd_any(const FftGeom &tile, const FwdFftArgs &a, bool compute_f32, const FftLaunch &cfg,
                   const void *tw, const void *twM, const void *hM, hipStream_t s) {
  if (compute_f32) {
    if (a.src_f32) return fwd<float, float, false, BLUE>(tile, a, cfg, tw, twM, hM, s);
    return fwd<float, double, false, BLUE>(tile, a, cfg, tw, twM, hM, s);
  }
  if (a.src_f32) return fwd<double, float, false, BLUE>(tile, a, cfg, tw, twM, hM, s);
  if (a.round_f32) return fwd<double, double, true, BLUE>(tile, a, cfg, tw, twM, hM, s);
  return fwd<double, double, false, BLUE>(tile, a, cfg, tw, twM, hM, s);
}

template <bool BLUE>
hipError_t inv_any(const FftGeom &tile, const InvFftArgs &a, bool compute_f32, const FftLaunch &cfg,
                   const void *tw, const void *twM, const void *hM, hipStream_t s) {
  if (compute_f32) {
    if (a.src_f32) return inv<float, float, BLUE>(tile, a, cfg, tw, twM, hM, s);
    return inv<float, double, BLUE>(tile, a, cfg, tw, twM, hM, s);
  }
  if (a.src_f32) return inv<double, float, BLUE>(tile, a, cfg, tw, twM, hM, s);
  return inv<double, double, BLUE>(tile, a, cfg, tw, twM, hM, s);
}

}  // namespace

// Generic launches, one translation unit each (fft_generic_*.hip) so that
// they compile in parallel; the Bluestein ones take the M-point tables.
hipError_t generic_forward(const FftGeom &tile, const FwdFftArgs &a, bool compute_f32, const FftLaunch &cfg,
                     const void *tw, hipStream_t s);
hipError_t generic_forward_blue(const FftGeom &tile, const FwdFftArgs &a, bool compute_f32, const FftLaunch &cfg,
                          const void *tw, const void *twM, const void *hM, hipStream_t s);
hipError_t generic_inverse(const FftGeom &tile, const InvFftArgs &a, bool compute_f32, const FftLaunch &cfg,
                     const void *tw, hipStream_t s);
hipError_t generic_inverse_blue(const FftGeom &tile, const InvFftArgs &a, bool compute_f32, const FftLaunch &cfg,
                          const void *tw, const void *twM, const void *hM, hipStream_t s);

}  // namespace fftmv

