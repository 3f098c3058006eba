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

// Each thread copies V consecutive columns (one 16-byte load of double
// pairs, or an 8-byte load of float pairs, when V = 2) of kRowsPerBlock
// rows; consecutive lanes touch consecutive addresses on both sides.
constexpr int kRowsPerBlock = 4;

template <typename S, typename D, int V>
__global__ __launch_bounds__(kBlock) void cast_kernel(const S *__restrict__ src, int64_t lds, D *__restrict__ dst,
                                                      int64_t ldd, int64_t rows, int64_t cols) {
  const int64_t c = (static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x) * V;
  if (c >= cols) return;
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * kRowsPerBlock;
  const int64_t r1 = r0 + kRowsPerBlock < rows ? r0 + kRowsPerBlock : rows;
  if constexpr (V == 2) {
    typedef S S2 __attribute__((ext_vector_type(2)));
    typedef D D2 __attribute__((ext_vector_type(2)));
    if (c + 1 < cols) {
      S2 in[kRowsPerBlock];
#pragma unroll
      for (int i = 0; i < kRowsPerBlock; ++i)
        if (r0 + i < r1) in[i] = *reinterpret_cast<const S2 *>(src + (r0 + i) * lds + c);
#pragma unroll
      for (int i = 0; i < kRowsPerBlock; ++i)
        if (r0 + i < r1)
          *reinterpret_cast<D2 *>(dst + (r0 + i) * ldd + c) = D2{static_cast<D>(in[i].x), static_cast<D>(in[i].y)};
      return;
    }
  }
  for (int64_t r = r0; r < r1; ++r) dst[r * ldd + c] = static_cast<D>(src[r * lds + c]);  // last odd column
}

template <typename S, typename D>
void cast(const CastArgs &a, hipStream_t s) {
  // pairs when both row strides are even and both bases are aligned to a pair
  const bool pairs = (a.lds % 2 == 0) && (a.ldd % 2 == 0) && (reinterpret_cast<uintptr_t>(a.src) % (2 * sizeof(S)) == 0) &&
                     (reinterpret_cast<uintptr_t>(a.dst) % (2 * sizeof(D)) == 0);
  const int v = pairs ? 2 : 1;
  const int64_t per = static_cast<int64_t>(kBlock) * v;
  const dim3 grid(static_cast<unsigned>((a.cols + per - 1) / per),
                  static_cast<unsigned>((a.rows + kRowsPerBlock - 1) / kRowsPerBlock));
  if (pairs)
    hipLaunchKernelGGL((cast_kernel<S, D, 2>), grid, dim3(kBlock), 0, s, static_cast<const S *>(a.src), a.lds,
                       static_cast<D *>(a.dst), a.ldd, a.rows, a.cols);
  else
    hipLaunchKernelGGL((cast_kernel<S, D, 1>), grid, dim3(kBlock), 0, s, static_cast<const S *>(a.src), a.lds,
                       static_cast<D *>(a.dst), a.ldd, a.rows, a.cols);
}

}  // namespace

hipError_t launch_cast(const CastArgs &a, hipStream_t s) {
  if (a.rows <= 0 || a.cols <= 0) return hipSuccess;
  if ((a.rows + kRowsPerBlock - 1) / kRowsPerBlock > 65535) return hipErrorInvalidValue;
  if (a.src_f32 && a.dst_f32)
    cast<float, float>(a, s);
  else if (a.src_f32)
    cast<float, double>(a, s);
  else if (a.dst_f32)
    cast<double, float>(a, s);
  else
    cast<double, double>(a, s);
  return hipGetLastError();
}

}  // namespace fftmv
