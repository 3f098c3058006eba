// Generic inverse batched real FFT in Bluestein (chirp-z) form, for lengths
// without a radix schedule (see fft_generic.hpp).
#include "fft_generic.hpp"

namespace fftmv {

hipError_t generic_inverse_blue(const FftGeom &tile, const InvFftArgs &a, bool compute_f32, const FftLaunch &cfg,
                          const void *tw, const void *twM, const void *hM, hipStream_t s) {
  return inv_any<true>(tile, a, compute_f32, cfg, tw, twM, hM, s);
}

}  // namespace fftmv
