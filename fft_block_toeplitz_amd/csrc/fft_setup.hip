// The setup transform of "Mixed-precision FFTMatvec performance optimization
// on AMD GPUs", section 1.1: the frequency blocks Fhat_k of F, every
// (row, column) series zero-padded to 2 Nt and transformed in FP64 once
// (the c_F eps_d term of the error bound), for Nt = 1000 and Nt = 2000 and
// batches of at least kWideBatch channels.
//
// F is [Nt][Nd Nm] (channels fastest), so a workgroup takes C adjacent
// channels and every time step of its tile is one run of 8 C bytes. The
// plain tile (the whole length-Nt complex transform of C channels in LDS)
// fits only 8 FP64 channels at Nt = 1000 and 4 at Nt = 2000; this kernel
// splits the transform so that a tile of 16 (Nt = 1000) or 8 (Nt = 2000)
// channels needs a quarter of it at a time.
//
// With the even/odd packing z[n] = x[2n] + i x[2n+1] the real transform of
// length 2L (L = Nt) is carried by the complex length-L transform Z of z,
// and z[n] = 0 for n >= L/2 (the zero pad). Write L = R1 * 125 (R1 = 8 or
// 16) and n = n2 + 125 n1. One decimation-in-frequency step gives R1
// independent 125-point transforms:
//   Z[s + R1 k2] = sum_n2 W_125^(n2 k2) y_s[n2],
//   y_s[n2] = W_L^(n2 s) sum_{n1 < R1/2} z[n2 + 125 n1] W_R1^(n1 s)
// (only R1/2 terms: the rest of z is the pad). The real bins need Z[k] with
// Z[L - k]; L - k lies in slot R1 - s (slot 0 and slot R1/2 mirror onto
// themselves), so the slots are taken in mirror-closed groups {0, R1/2},
// {g, R1 - g}: NSL slots per round, in LDS as [125 rows][NSL slots][C].
// Each thread keeps its butterflies' R1/2 packed samples in registers from
// one load phase to the last round (every sample of F read once), writes
// the round's y_s into LDS, the three radix-5 Stockham passes follow, and
// each mirror pair of bins leaves together:
//   X[k] = E + T, X[L - k] = conj(E - T),
//   E = (Z[k] + conj Z[L-k]) / 2, T = -i/2 (Z[k] - conj Z[L-k]) w_2L^k.
// Measured on MI355X (transform alone; plain 8- and 4-channel tiles:
// 3.50 and 38.5 ms): Main (Nm = 5000, Nd = 100, Nt = 1000) 3.00 ms, the
// Scale share (Nm = 20000, Nd = 100, Nt = 2000) 28.4 ms.
#include "fft_fixed.hpp"

namespace fftmv {
namespace {

constexpr int kSub = 125;  // length of the sub-transforms: 5 x 5 x 5

// cos(j pi / 8) for any integer j (the angles of W_8 and W_16)
constexpr double kCosPi8[5] = {1.0, 0.92387953251128675613, 0.70710678118654752440, 0.38268343236508977173, 0.0};
constexpr double cos_pi8(int j) {
  j = ((j % 16) + 16) % 16;
  if (j > 8) j = 16 - j;
  return j > 4 ? -kCosPi8[8 - j] : kCosPi8[j];
}
constexpr double sin_pi8(int j) { return cos_pi8(4 - j); }

// A += z exp(-i J pi/8), B += z exp(+i J pi/8); quarter turns cost no
// multiplication
template <int J>
__device__ __forceinline__ void rot_acc(cx<double> &A, cx<double> &B, cx<double> z) {
  constexpr int j = ((J % 16) + 16) % 16;
  if constexpr (j == 0) {
    A = A + z;
    B = B + z;
  } else if constexpr (j == 8) {
    A = A - z;
    B = B - z;
  } else if constexpr (j == 4) {
    A = A + mk(z.im, -z.re);
    B = B + mk(-z.im, z.re);
  } else if constexpr (j == 12) {
    A = A + mk(-z.im, z.re);
    B = B + mk(z.im, -z.re);
  } else {
    constexpr double c = cos_pi8(j), s = sin_pi8(j);
    A = mk(A.re + (z.re * c + z.im * s), A.im + (z.im * c - z.re * s));
    B = mk(B.re + (z.re * c - z.im * s), B.im + (z.im * c + z.re * s));
  }
}

template <int R1, int H, int G, int N>
__device__ __forceinline__ void rot_terms(const cx<double> (&z)[H], cx<double> &A, cx<double> &B) {
  if constexpr (N < H) {
    rot_acc<N * G * (16 / R1)>(A, B, z[N]);
    rot_terms<R1, H, G, N + 1>(z, A, B);
  }
}

// The two sums of mirror group G: A = sum_n1 z[n1] W_R1^(n1 G) and
// B = sum_n1 z[n1] W_R1^(-n1 G) (slots G and R1 - G); for G = 0 the slots
// 0 and R1/2: A = sum z[n1], B = sum (-1)^n1 z[n1].
// CROT: the rotations as compile-time constants; else from the table.
template <int R1, int H, int G, bool CROT, int L>
__device__ __forceinline__ void group_sums(const cx<double> (&z)[H], const cx<double> *__restrict__ tw, cx<double> &A,
                                           cx<double> &B) {
  A = z[0];
  B = z[0];
  if constexpr (G == 0) {
#pragma unroll
    for (int n1 = 1; n1 < H; ++n1) {
      A = A + z[n1];
      B = (n1 & 1) ? B - z[n1] : B + z[n1];
    }
  } else if constexpr (CROT) {
    rot_terms<R1, H, G, 1>(z, A, B);
  } else {
#pragma unroll
    for (int n1 = 1; n1 < H; ++n1) {
      const cx<double> w = tw[(2 * L / R1) * ((n1 * G) % R1)];  // W_R1^(n1 G) = w_2L^(250 (n1 G mod R1))
      A = A + cmul(z[n1], w);
      B = B + cmulc(z[n1], w);
    }
  }
}

template <int R1, int H, int GG, int NG, bool CROT, int L>
__device__ __forceinline__ void group_sums_of(int g, const cx<double> (&z)[H], const cx<double> *__restrict__ tw,
                                              cx<double> &A, cx<double> &B) {
  if constexpr (GG < NG) {
    if (g == GG) group_sums<R1, H, GG, CROT, L>(z, tw, A, B);
    else group_sums_of<R1, H, GG + 1, NG, CROT, L>(g, z, tw, A, B);
  }
}

// L = Nt (1000 or 2000), C channels per workgroup, NSL slots per round,
// NTS: streamed (non-temporal) spectrum stores; CROT: see group_sums.
// Addresses are 64-bit (32-bit lane offsets from uniform bases measured no
// faster). The output: channel ch goes to row ch / cpr, column ch % cpr of its
// frequency's block (dst32 complex64 and/or dst64 complex128).
template <int L, int C, int TPB, int NSL, bool NTS, bool CROT>
__global__ __launch_bounds__(TPB) void rfft_setup_dif(FwdFftArgs a, const cx<double> *__restrict__ tw,
                                                      int64_t ntiles) {
  constexpr int R1 = L / kSub, H = R1 / 2, NG = R1 / 2;
  static_assert(R1 * kSub == L && R1 % 2 == 0 && NSL % 2 == 0 && NG % (NSL / 2) == 0, "mirror groups per round");
  static_assert((kSub - 1) * R1 < L, "twiddle indices 2 n2 s stay below 2L");
  constexpr int NROUND = NG / (NSL / 2);
  constexpr int CC = C * NSL;  // LDS columns: [row][slot][channel]
  constexpr int NB0 = kSub * C, B0 = (NB0 + TPB - 1) / TPB;
  constexpr int TWM = L / kSub;  // the table is w_2L; the 125-point passes step it by 2L / 250
  __shared__ cx<double> lds[kSub * CC];

  const int64_t tile = xcd_contiguous_block(blockIdx.x, ntiles);
  const char *src = static_cast<const char *>(a.src);
  const int64_t ld = a.src_ld;

  // the packed samples z[n2 + 125 n1], n1 < H, of this thread's butterflies
  // (channel b % C, n2 = b / C): rows 2 n and 2 n + 1 of F
  cx<double> z[B0][H];
#pragma unroll
  for (int i = 0; i < B0; ++i) {
    const int b = threadIdx.x + i * TPB;
    const int c = b % C, n2 = b / C;
    const int64_t ch = tile * C + c;
    const bool live = (NB0 % TPB == 0 || b < NB0) && ch < a.nchan;
    const int64_t lane = (2 * static_cast<int64_t>(n2) * ld + ch) * 8;
#pragma unroll
    for (int n1 = 0; n1 < H; ++n1) {
      const char *b0 = src + static_cast<int64_t>(2 * kSub * n1) * ld * 8, *b1 = b0 + ld * 8;
      z[i][n1] = live ? mk(*reinterpret_cast<const double *>(b0 + lane), *reinterpret_cast<const double *>(b1 + lane))
                      : mk(0.0, 0.0);
    }
  }

  // output positions of this thread's channel pair (c0, c0 + 1): fixed,
  // since TPB is a multiple of C / 2; the second channel may start the
  // next row of the block
  constexpr int CP = C / 2;
  static_assert(TPB % CP == 0, "channel pair fixed per thread");
  const int c0 = (threadIdx.x % CP) * 2;
  const int64_t ch0 = tile * C + c0;
  const bool first = ch0 < a.nchan, second = ch0 + 1 < a.nchan;
  cx<float> *p32a = nullptr, *p32b = nullptr;
  cx<double> *p64a = nullptr, *p64b = nullptr;
  bool two = false;  // one 16-byte complex64 store for both channels
  if (first) {
    const int64_t row = ch0 / a.cpr, col = ch0 - row * a.cpr;
    int64_t row1 = row, col1 = col + 1;
    if (second && col1 == a.cpr) {
      row1 = row + 1;
      col1 = 0;
    }
    if (a.dst32) {
      p32a = static_cast<cx<float> *>(a.dst32) + row * a.ldr32 + col;
      p32b = static_cast<cx<float> *>(a.dst32) + row1 * a.ldr32 + col1;
      two = second && row1 == row && ((row * a.ldr32 + col) & 1) == 0;
    }
    if (a.dst64) {
      p64a = static_cast<cx<double> *>(a.dst64) + row * a.ldr64 + col;
      p64b = static_cast<cx<double> *>(a.dst64) + row1 * a.ldr64 + col1;
    }
  }
  auto put = [&](int k, cx<double> x0, cx<double> x1) {
    if (p32a) {
      const int64_t o = k * a.fstride32;
      if (two) {
        store_pair<NTS>(p32a + o, cvt<float>(x0), cvt<float>(x1));
      } else {
        store_one<NTS>(p32a + o, cvt<float>(x0));
        if (second) store_one<NTS>(p32b + o, cvt<float>(x1));
      }
    }
    if (p64a) {
      const int64_t o = k * a.fstride64;
      store_one<NTS>(p64a + o, x0);
      if (second) store_one<NTS>(p64b + o, x1);
    }
  };

#pragma unroll
  for (int r = 0; r < NROUND; ++r) {
    // y of the round's slots into LDS
#pragma unroll
    for (int i = 0; i < B0; ++i) {
      const int b = threadIdx.x + i * TPB;
      if (NB0 % TPB == 0 || b < NB0) {
        const int c = b % C, n2 = b / C;
#pragma unroll
        for (int gi = 0; gi < NSL / 2; ++gi) {
          const int g = r * (NSL / 2) + gi;  // a constant once the loops unroll
          cx<double> A, B;
          group_sums_of<R1, H, 0, NG, CROT, L>(g, z[i], tw, A, B);
          cx<double> ya, yb;
          if (g == 0) {
            ya = A;
            yb = cmul(B, tw[n2 * R1]);  // W_L^(n2 R1/2)
          } else {
            ya = cmul(A, tw[2 * n2 * g]);         // W_L^(n2 g)
            yb = cmul(B, tw[2 * n2 * (R1 - g)]);  // W_L^(n2 (R1 - g))
          }
          lds[n2 * CC + (2 * gi) * C + c] = ya;
          lds[n2 * CC + (2 * gi + 1) * C + c] = yb;
        }
      }
    }
    __syncthreads();
    // the 125-point transforms of the NSL slots x C channels
    ct_lds_pass<double, kSub, CC, TPB, 0, -1, TWM, false>(lds, tw);
    ct_lds_pass<double, kSub, CC, TPB, 1, -1, TWM, false>(lds, tw);
    ct_lds_pass<double, kSub, CC, TPB, 2, -1, TWM, false>(lds, tw);
    // the mirror pairs of bins: group 0 first (126 items: slot 0 with
    // k2 = 0..62 against (125 - k2) mod 125, which gives bins 0 and L at
    // k2 = 0; slot R1/2 with k2 = 0..62 against 124 - k2, where k2 = 62 is
    // bin L/2 paired with itself), then 125 per further group (slot g at k2
    // against slot R1 - g at 124 - k2)
    const int nitems = (NSL / 2) * kSub + (r == 0 ? 1 : 0);
    if (first) {
      for (int b = threadIdx.x; b < nitems * CP; b += TPB) {
        int it = b / CP;
        int sla, k2a, slb, k2b, k;
        if (r == 0 && it < 2 * 63) {
          if (it < 63) {
            sla = slb = 0;
            k2a = it;
            k2b = it == 0 ? 0 : kSub - it;
            k = R1 * it;
          } else {
            sla = slb = 1;
            k2a = it - 63;
            k2b = kSub - 1 - k2a;
            k = R1 / 2 + R1 * k2a;
          }
        } else {
          if (r == 0) it -= 1;  // group 0 took one item more than kSub
          const int gi = it / kSub;
          k2a = it - gi * kSub;
          sla = 2 * gi;
          slb = 2 * gi + 1;
          k2b = kSub - 1 - k2a;
          k = r * (NSL / 2) + gi + R1 * k2a;
        }
        const cx<double> w = tw[k];
        cx<double> xa[2], xb[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const cx<double> za = lds[k2a * CC + sla * C + c0 + e], zb = conj(lds[k2b * CC + slb * C + c0 + e]);
          const cx<double> ev = scale(za + zb, 0.5), dd = za - zb;
          const cx<double> t = cmul(mk(dd.im * 0.5, -dd.re * 0.5), w);
          xa[e] = ev + t;
          xb[e] = conj(ev - t);
        }
        put(k, xa[0], xa[1]);
        if (2 * k != L) put(L - k, xb[0], xb[1]);
      }
    }
    if (r + 1 < NROUND) __syncthreads();  // the next round overwrites the LDS tile
  }
}

// Tiles: Nt = 1000, 16 channels (every time step of F and every bin row of
// a 16-channel block is one 128-byte line), 2 slots per round (64 KB of
// LDS), rotations as constants, cached stores; Nt = 2000, 8 channels,
// 4 slots per round (64 KB), rotations from the table (as constants the
// 8-term sums spill registers), streamed stores. Both in 1024 threads, one
// workgroup per CU. Measured against other shapes of the same kernel:
// Nt = 1000 with 8 channels in 512 threads (two workgroups per CU)
// 3.33 ms; Nt = 2000 with 2 slots per round 32.3 ms, cached stores 29.3.
template <int L>
struct SetupTile;
template <>
struct SetupTile<1000> {
  static constexpr int C = 16, TPB = 1024, NSL = 2;
  static constexpr bool NTS = false, CROT = true;
};
template <>
struct SetupTile<2000> {
  static constexpr int C = 8, TPB = 1024, NSL = 4;
  static constexpr bool NTS = true, CROT = false;
};

template <int L>
hipError_t launch_setup(const FwdFftArgs &a, const void *tw, hipStream_t s) {
  using T = SetupTile<L>;
  const int64_t ntiles = (a.nchan + T::C - 1) / T::C;
  if (!grid_fits(ntiles, T::TPB)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((rfft_setup_dif<L, T::C, T::TPB, T::NSL, T::NTS, T::CROT>), dim3(static_cast<unsigned>(ntiles)),
                     dim3(T::TPB), 0, s, a, static_cast<const cx<double> *>(tw), ntiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fft_setup_wide(int L, const FwdFftArgs &a, const void *tw, hipStream_t s) {
  if (a.Nt != L || a.src_f32 || a.round_f32 || a.nchan < 1 || a.nchan > a.src_ld || a.cpr < 1)
    return hipErrorInvalidValue;
  if (L == 1000) return launch_setup<1000>(a, tw, s);
  if (L == 2000) return launch_setup<2000>(a, tw, s);
  return hipErrorInvalidValue;
}

}  // namespace fftmv
