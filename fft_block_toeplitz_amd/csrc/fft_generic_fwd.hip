// Generic forward batched real FFT (runtime length and schedule; see
// fft_generic.hpp), radix form, and the host-side launch of every forward
// transform (fixed-length kernels first, then radix, then Bluestein form),
// with the launch configuration shared by all generic transforms.
#include "fft_generic.hpp"

namespace fftmv {

// Channels per workgroup (C = 0 when the transform does not fit): the widest tile that still leaves at least
// kMinFftBlocks workgroups (one per CU), else the narrowest tile that fits
// (small batches). Wide tiles read and write each time step and frequency
// in runs of C channels, where one channel per workgroup reads every cache
// line once per channel. The workgroup has 1024 threads (half the registers
// per thread, more LDS) when 256 threads cannot hold a pass's butterflies,
// or when there are fewer than two workgroups per CU: a 256-thread
// workgroup then leaves each CU with 4 to 8 waves to hide memory latency.
// Measured at Nt = 256, 1009 (Bluestein), 1024 and 1029, 128 to 8192
// channels, FP32 and FP64.
constexpr int64_t kMinFftBlocks = 256;

FftLaunch fft_launch_config(const FftGeom &g, bool f32, int64_t nchan) {
  const int64_t esz = f32 ? 8 : 16;
  auto fits = [&](int C, int tpb) {
    const int64_t lds_cap = tpb == kBlockWide ? kMaxLdsWide : kMaxLds;
    const int vmax = tpb == kBlockWide ? kVmaxWide : kVmax;
    if (static_cast<int64_t>(g.L) * C * esz > lds_cap) return false;
    for (int p = 0; p < g.npass; ++p) {
      const int64_t nb = static_cast<int64_t>(g.L / g.radix[p]) * C;
      if (nb > static_cast<int64_t>(vmax / g.radix[p]) * tpb) return false;
    }
    return true;
  };
  auto cfg = [](int C, bool wide) {
    return FftLaunch{C, wide ? kVmaxWide : kVmax, wide ? kBlockWide : kBlock};
  };
  FftLaunch narrowest;
  for (int C = kMaxChannelsPerBlock; C >= 1; C >>= 1) {
    const bool f256 = fits(C, kBlock), f1024 = fits(C, kBlockWide);
    if (!f256 && !f1024) continue;
    const int64_t nblocks = (nchan + C - 1) / C;
    if (nblocks >= kMinFftBlocks) return cfg(C, f1024 && (!f256 || nblocks < 2 * kMinFftBlocks));
    narrowest = cfg(C, !f256);
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

hipError_t generic_forward(const FftGeom &tile, const FwdFftArgs &a, bool compute_f32, const FftLaunch &cfg,
                     const void *tw, hipStream_t s) {
  return fwd_any<false>(tile, a, compute_f32, cfg, tw, nullptr, nullptr, s);
}

hipError_t launch_fft_forward(const FftGeom &g, const FwdFftArgs &a, bool compute_f32, const void *tw,
                              hipStream_t s, const BlueTables *blue) {
  hipError_t fixed_err = hipSuccess;
  if (!blue && launch_fft_forward_fixed(g, a, compute_f32, tw, s, &fixed_err))
    return fixed_err != hipSuccess ? fixed_err : hipGetLastError();
  const FftGeom &tile = blue ? blue->gM : g;
  const FftLaunch cfg = fft_launch_config(tile, compute_f32, a.nchan);
  if (cfg.C == 0) return hipErrorInvalidValue;
  if (!grid_fits((a.nchan + cfg.C - 1) / cfg.C, cfg.tpb)) return hipErrorInvalidConfiguration;
  if (blue) {
    const void *twM = compute_f32 ? blue->tw32 : blue->tw64, *hM = compute_f32 ? blue->hf32 : blue->hf64;
    if (!twM || !hM) return hipErrorInvalidValue;
    const hipError_t e = generic_forward_blue(tile, a, compute_f32, cfg, tw, twM, hM, s);
    if (e != hipSuccess) return e;
  } else {
    const hipError_t e = generic_forward(tile, a, compute_f32, cfg, tw, s);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

}  // namespace fftmv
