// Generic forward batched real FFT (runtime length and schedule; see
// fft_generic.hpp), radix form, and the host-side launch of every forward
// transform (fixed-length kernels first, then radix, then Bluestein form),
// with the launch configuration shared by all generic transforms.
#include "fft_generic.hpp"

namespace fftmv {

// Channels per workgroup for a schedule, precision and batch: the widest C
// that still gives at least 1024 workgroups (four per CU); for small batches
// the narrowest C (most workgroups). C = 0 when the transform does not fit.
FftLaunch fft_launch_config(const FftGeom &g, bool f32, int64_t nchan) {
  const int64_t esz = f32 ? 8 : 16;
  auto fits = [&](int C) {
    if (static_cast<int64_t>(g.L) * C * esz > kMaxLds) return false;
    for (int p = 0; p < g.npass; ++p) {
      const int64_t nb = static_cast<int64_t>(g.L / g.radix[p]) * C;
      if (nb > static_cast<int64_t>(kVmax / g.radix[p]) * kBlock) return false;
    }
    return true;
  };
  FftLaunch narrowest;
  for (int C = kMaxChannelsPerBlock; C >= 1; C >>= 1) {
    if (!fits(C)) continue;
    if ((nchan + C - 1) / C >= 1024) return {C, kVmax};
    narrowest = {C, kVmax};
  }
  return narrowest;
}

int fft_channels_per_block(const FftGeom &g, bool f32, int64_t nchan) { return fft_launch_config(g, f32, nchan).C; }

int64_t bluestein_length(int64_t L) {
  if (L < 2 || L > (int64_t(1) << 20) || make_geometry(static_cast<int>(L)).L == L) return 0;
  int64_t M = 1;
  while (M < 2 * L - 1) M *= 2;
  const FftGeom gM = make_geometry(static_cast<int>(M));
  if (fft_channels_per_block(gM, false, 1) == 0 || fft_channels_per_block(gM, true, 1) == 0) return 0;
  return M;
}

void generic_forward(const FftGeom &tile, const FwdFftArgs &a, bool compute_f32, const FftLaunch &cfg,
                     const void *tw, hipStream_t s) {
  fwd_any<false>(tile, a, compute_f32, cfg, tw, nullptr, nullptr, s);
}

hipError_t launch_fft_forward(const FftGeom &g, const FwdFftArgs &a, bool compute_f32, const void *tw,
                              hipStream_t s, const BlueTables *blue) {
  if (!blue && launch_fft_forward_fixed(g, a, compute_f32, tw, s)) return hipGetLastError();
  const FftGeom &tile = blue ? blue->gM : g;
  const FftLaunch cfg = fft_launch_config(tile, compute_f32, a.nchan);
  if (cfg.C == 0 || (a.nchan + cfg.C - 1) / cfg.C > INT32_MAX) return hipErrorInvalidValue;
  if (blue) {
    const void *twM = compute_f32 ? blue->tw32 : blue->tw64, *hM = compute_f32 ? blue->hf32 : blue->hf64;
    if (!twM || !hM) return hipErrorInvalidValue;
    generic_forward_blue(tile, a, compute_f32, cfg, tw, twM, hM, s);
  } else {
    generic_forward(tile, a, compute_f32, cfg, tw, s);
  }
  return hipGetLastError();
}

}  // namespace fftmv
