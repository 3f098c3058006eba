// Inverse batched real FFT with the unpad folded in (stages 4-5) of
// "Mixed-precision FFTMatvec performance optimization on AMD GPUs",
// section 1.1, specialised for Nt = 1000 and Nt = 2000.
#include "fft_fixed.hpp"

namespace fftmv {
namespace {

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
         fits_32bit(a.Nt, a.dst_ld, 8) && a.nchan <= a.src_ld && a.nchan <= a.dst_ld &&
         grid_fits(a.nchan, kCtItemsPerChannel);
}


}  // namespace

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
