// Batched real FFTs specialised for one transform length (stages 2 and 4
// of "Mixed-precision FFTMatvec performance optimization on AMD GPUs",
// section 1.1, for the configured workloads Nt = 1000 and Nt = 2000):
// the pieces shared by the forward (fft_fixed_fwd.hip) and inverse
// (fft_fixed_inv.hip) kernels. Same algorithm as the generic kernels in
// fft_generic.hpp; here the schedule, butterfly counts and divisors are
// compile-time constants.
#pragma once

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

// index of element n of column c in a tile of C columns, padded (above) or not
template <int C, bool PAD>
__device__ __forceinline__ int ct_at(int n, int c) {
  return PAD ? ct_idx<C>(n, c) : n * C + c;
}

// One Stockham pass (P > 0 has twiddles) over C columns of length-L
// transforms in LDS. The twiddle table holds w_M^t with M = 2 L TWM (the
// plan's table of a longer transform when TWM > 1).
template <typename T, int L, int C, int TPB, int P, int S, int TWM = 1, bool PAD = true>
__device__ __forceinline__ void ct_lds_pass(cx<T> *lds, const cx<T> *__restrict__ tw) {
  constexpr FftGeom g = make_geometry(L);
  constexpr int R = g.radix[P], NS = g.ns[P], TWS = g.twstep[P] * TWM;
  constexpr int Lr = L / R, NB = Lr * C, B = (NB + TPB - 1) / TPB;
  cx<T> v[B][R];
#pragma unroll
  for (int i = 0; i < B; ++i) {
    const int b = threadIdx.x + i * TPB;
    if (NB % TPB == 0 || b < NB) {
      const int c = b % C, j = b / C;
#pragma unroll
      for (int q = 0; q < R; ++q) v[i][q] = lds[ct_at<C, PAD>(j + q * Lr, c)];
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
      for (int q = 0; q < R; ++q) lds[ct_at<C, PAD>(base + q * NS, c)] = v[i][q];
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
// Wider tile of the forward FP64 transform at Nt = 1000 for large batches:
// 8 channels in 1024 threads (144 KB of LDS, one workgroup per CU), so each
// time step of the FP64 input is read in 64-byte runs instead of 32.
// Measured (5000 channels): 50.7 us against 68.1 with 4 x 512; it wins from
// 2048 channels (19.1 against 28.7 us) and loses at 1024 (11.8 against
// 10.4). The inverse reads complex128 (64-byte runs at 4 channels already)
// and stays at 4 x 512.
template <typename T>
constexpr CtTile ct_wider_fwd_tile(int L) {
  return sizeof(T) == 8 && L == 1000 ? CtTile{8, 1024} : ct_wide_tile<T>(L);
}
constexpr int64_t kWiderBatch = 2048;
constexpr bool has_ct(int L) { return L == 1000 || L == 2000; }
// Work-items per channel of the widest-threaded tile above (4 channels in
// 1024 threads; one channel in 256): a batch whose grid fits at this rate
// fits with every tile; larger batches take the generic kernels.
constexpr int64_t kCtItemsPerChannel = 256;
// Channels from which the wide tile pays. Measured at Nt = 1000, forward
// and inverse, FP32 and FP64: one channel per workgroup wins below ~256
// channels (6.7 against 7.0 us) and collapses beyond ~1000, where its
// 8-byte column reads fetch each cache line once per channel (FP32 forward,
// 3072 channels: 120 us against 12.7; FP64, 2048: 96 against 29); from 512
// channels the wide tile is ahead in all four kernels.
constexpr int64_t kWideBatch = 512;

}  // namespace
}  // namespace fftmv
