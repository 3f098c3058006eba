// Generic inverse batched real FFT with the unpad folded in (runtime length
// and schedule; see fft_generic.hpp), radix form, and the host-side launch of
// every inverse transform (fixed-length kernels first, then radix, then
// Bluestein form).
#include "fft_generic.hpp"

namespace fftmv {

hipError_t generic_inverse(const FftGeom &tile, const InvFftArgs &a, bool compute_f32, const FftLaunch &cfg,
                     const void *tw, hipStream_t s) {
  return inv_any<false>(tile, a, compute_f32, cfg, tw, nullptr, nullptr, s);
}

hipError_t launch_fft_inverse(const FftGeom &g, const InvFftArgs &a, bool compute_f32, const void *tw,
                              hipStream_t s, const BlueTables *blue) {
  if (!blue && launch_fft_inverse_fixed(g, a, compute_f32, tw, s)) return hipGetLastError();
  const FftGeom &tile = blue ? blue->gM : g;
  const FftLaunch cfg = fft_launch_config(tile, compute_f32, a.nchan);
  if (cfg.C == 0) return hipErrorInvalidValue;
  if (!grid_fits((a.nchan + cfg.C - 1) / cfg.C, cfg.tpb)) return hipErrorInvalidConfiguration;
  if (blue) {
    const void *twM = compute_f32 ? blue->tw32 : blue->tw64, *hM = compute_f32 ? blue->hi32 : blue->hi64;
    if (!twM || !hM) return hipErrorInvalidValue;
    const hipError_t e = generic_inverse_blue(tile, a, compute_f32, cfg, tw, twM, hM, s);
    if (e != hipSuccess) return e;
  } else {
    const hipError_t e = generic_inverse(tile, a, compute_f32, cfg, tw, s);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

}  // namespace fftmv
