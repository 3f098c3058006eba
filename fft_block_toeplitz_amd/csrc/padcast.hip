// Stage 1 (broadcast + zero pad) and stage 5 (unpad + reduce) of
// "Mixed-precision FFTMatvec performance optimization on AMD GPUs",
// section 1.1, in their stand-alone form: a coalesced copy of the Nt live
// time steps with the precision change at the stage boundary. On one GPU
// broadcast and reduce are the identity; the zero half of the padded buffer
// is implicit (the forward FFT never reads it) and the inverse FFT only
// produces the Nt time steps the unpad keeps.
#include "common.hpp"
#include "internal.hpp"

namespace fftmv {
namespace {

// One workgroup row-segment of 256 consecutive columns per (blockIdx.x,
// blockIdx.y): consecutive lanes touch consecutive addresses on both sides.
template <typename S, typename D>
__global__ __launch_bounds__(kBlock) void cast_kernel(const S *__restrict__ src, int64_t lds, D *__restrict__ dst,
                                                      int64_t ldd, int64_t rows, int64_t cols) {
  const int64_t c = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (c >= cols) return;
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) dst[r * ldd + c] = static_cast<D>(src[r * lds + c]);
}

}  // namespace

hipError_t launch_cast(const CastArgs &a, hipStream_t s) {
  if (a.rows <= 0 || a.cols <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((a.cols + kBlock - 1) / kBlock),
                  static_cast<unsigned>(a.rows < 65535 ? a.rows : 65535));
  if (a.src_f32 && a.dst_f32)
    hipLaunchKernelGGL((cast_kernel<float, float>), grid, dim3(kBlock), 0, s, static_cast<const float *>(a.src), a.lds,
                       static_cast<float *>(a.dst), a.ldd, a.rows, a.cols);
  else if (a.src_f32)
    hipLaunchKernelGGL((cast_kernel<float, double>), grid, dim3(kBlock), 0, s, static_cast<const float *>(a.src),
                       a.lds, static_cast<double *>(a.dst), a.ldd, a.rows, a.cols);
  else if (a.dst_f32)
    hipLaunchKernelGGL((cast_kernel<double, float>), grid, dim3(kBlock), 0, s, static_cast<const double *>(a.src),
                       a.lds, static_cast<float *>(a.dst), a.ldd, a.rows, a.cols);
  else
    hipLaunchKernelGGL((cast_kernel<double, double>), grid, dim3(kBlock), 0, s, static_cast<const double *>(a.src),
                       a.lds, static_cast<double *>(a.dst), a.ldd, a.rows, a.cols);
  return hipGetLastError();
}

}  // namespace fftmv
