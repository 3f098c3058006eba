// Forward batched real FFT (stage 2, and the setup transform of F) of
// "Mixed-precision FFTMatvec performance optimization on AMD GPUs",
// section 1.1, specialised for Nt = 1000 and Nt = 2000.
#include "fft_fixed.hpp"

namespace fftmv {
namespace {

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
  // complex64 spectrum leaves as 16-byte stores
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

// Spectrum stores: non-temporal for tiles of several channels (whole 64-byte
// runs per bin); plain for one channel per workgroup, whose 8- or 16-byte
// bins share each cache line with the bins of neighbouring workgroups, so
// the partial lines merge in L2 instead of reaching HBM one by one
// (measured, 100 FP64 channels at Nt = 1000: 5.8 against 6.7 us).
template <typename T, int L, bool ROUND, typename Src, int C, int TPB = kBlock>
void launch_fwd_ct(const FwdFftArgs &a, const void *tw, hipStream_t s) {
  const int64_t nblocks = (a.nchan + C - 1) / C;
  hipLaunchKernelGGL((rfft_forward_ct<T, L, C, TPB, (C > 1), ROUND, false, Src>), dim3(static_cast<unsigned>(nblocks)),
                     dim3(TPB), 0, s, a, static_cast<const cx<T> *>(tw), nblocks);
}

template <typename T, int L, bool ROUND, typename Src = double>
void launch_fwd_ct_c(const FwdFftArgs &a, const void *tw, hipStream_t s) {
  constexpr CtTile w = ct_wide_tile<T>(L), x = ct_wider_fwd_tile<T>(L);
  if constexpr (x.C != w.C || x.tpb != w.tpb) {
    if (a.nchan >= kWiderBatch) {
      launch_fwd_ct<T, L, ROUND, Src, x.C, x.tpb>(a, tw, s);
      return;
    }
  }
  if (a.nchan >= kWideBatch)
    launch_fwd_ct<T, L, ROUND, Src, w.C, w.tpb>(a, tw, s);
  else
    launch_fwd_ct<T, L, ROUND, Src, 1>(a, tw, s);
}

// the frequency blocks (setup) of small batches: FP64 transform, one channel
// per workgroup, 64-bit offsets, rows of cpr channels, plain stores (wide
// batches take the decimation-in-frequency kernel of fft_setup.hip)
template <int L>
void launch_fwd_ct_setup_narrow(const FwdFftArgs &a, const void *tw, hipStream_t s) {
  hipLaunchKernelGGL((rfft_forward_ct<double, L, 1, kBlock, false, false, true>), dim3(static_cast<unsigned>(a.nchan)),
                     dim3(kBlock), 0, s, a, static_cast<const cx<double> *>(tw), a.nchan);
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
         fits_32bit(a.Nt, a.src_ld, 8) && a.nchan <= a.src_ld && grid_fits(a.nchan, kCtItemsPerChannel);
}

}  // namespace

bool launch_fft_forward_fixed(const FftGeom &g, const FwdFftArgs &a, bool compute_f32, const void *tw, hipStream_t s,
                              hipError_t *err) {
  *err = hipSuccess;
  if (!fwd_ct_applies(g, a)) {
    // the frequency blocks: FP64 input and transform, any row structure and size
    const bool setup = has_ct(g.L) && a.Nt == g.L && !a.src_f32 && !a.round_f32 && !compute_f32 &&
                       a.nchan <= a.src_ld && a.cpr >= 1 && grid_fits(a.nchan, kCtItemsPerChannel);
    if (!setup) return false;
    if (a.nchan >= kWideBatch)
      *err = launch_fft_setup_wide(g.L, a, tw, s);
    else if (g.L == 1000)
      launch_fwd_ct_setup_narrow<1000>(a, tw, s);
    else
      launch_fwd_ct_setup_narrow<2000>(a, tw, s);
    return true;
  }
  if (g.L == 1000)
    launch_fwd_ct_any<1000>(a, compute_f32, tw, s);
  else
    launch_fwd_ct_any<2000>(a, compute_f32, tw, s);
  return true;
}

}  // namespace fftmv
