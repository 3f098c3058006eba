// Memory-system ceilings of the GPU, measured with plain kernels built from
// this repository: the context the benchmark reports next to the kernels'
// own bandwidth. Not part of the fftmv library (a separate shared object
// that only the benchmark loads).
//
//   ceiling_read       each workgroup streams one contiguous chunk of a
//                      buffer with every 16-byte load in flight (the best
//                      read rate an HBM-bound kernel can hope for)
//   ceiling_copy       the same chunks read and written back elsewhere
//   ceiling_tile_rw    the memory pattern of the setup transform without its
//                      arithmetic: a workgroup reads C adjacent FP64
//                      channels of every row of a [rows][nchan] array (runs
//                      of 8 C bytes) and writes rows + 1 rows of C 8-byte
//                      values at the same positions of an output array
//
// Each call launches one pass and returns a hipError_t; the caller times
// the launches with events on the same stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kTpb = 256;

// U 16-byte loads per thread, all in flight; chunk = kTpb * U * 16 bytes
template <int U>
__global__ __launch_bounds__(kTpb) void read_chunk(const f32x4 *__restrict__ p, int64_t n16, float *sink) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kTpb * U + threadIdx.x;
  f32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + static_cast<int64_t>(u) * kTpb;
    v[u] = i < n16 ? __builtin_nontemporal_load(p + i) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < U; ++u) s += v[u].x + v[u].y + v[u].z + v[u].w;
  if (s == 1234.5f) sink[threadIdx.x] = s;  // keeps the loads; never true for the zero-filled buffers used
}

template <int U>
__global__ __launch_bounds__(kTpb) void copy_chunk(const f32x4 *__restrict__ p, f32x4 *__restrict__ q, int64_t n16) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kTpb * U + threadIdx.x;
  f32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + static_cast<int64_t>(u) * kTpb;
    v[u] = i < n16 ? __builtin_nontemporal_load(p + i) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + static_cast<int64_t>(u) * kTpb;
    if (i < n16) q[i] = v[u];
  }
}

// C channels x rows per workgroup, 1024 threads: thread -> channel tid % C,
// rows tid / C + j * (1024 / C); then rows + 1 output rows of C values.
template <int C, int ROWS>
__global__ __launch_bounds__(1024) void tile_rw(const double *__restrict__ src, double *__restrict__ dst,
                                                int64_t nchan) {
  constexpr int RG = 1024 / C, PER = (ROWS + RG - 1) / RG;
  const int c = threadIdx.x % C, rg = threadIdx.x / C;
  const int64_t ch = static_cast<int64_t>(blockIdx.x) * C + c;
  double v[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int t = rg + j * RG;
    v[j] = t < ROWS ? __builtin_nontemporal_load(src + t * nchan + ch) : 0.0;
  }
  double s = 0.0;
#pragma unroll
  for (int j = 0; j < PER; ++j) s += v[j];
  for (int t = rg; t <= ROWS; t += RG) dst[t * nchan + ch] = s + t;
}

}  // namespace

extern "C" {

__attribute__((visibility("default"))) int ceiling_read(const void *buf, size_t bytes, int chunk_kib, void *sink,
                                                        hipStream_t s) {
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  if (!buf || !sink || n16 < 1) return static_cast<int>(hipErrorInvalidValue);
  const f32x4 *p = static_cast<const f32x4 *>(buf);
  if (chunk_kib == 64) {
    const int64_t nb = (n16 + kTpb * 16 - 1) / (kTpb * 16);
    hipLaunchKernelGGL(read_chunk<16>, dim3(static_cast<unsigned>(nb)), dim3(kTpb), 0, s, p, n16,
                       static_cast<float *>(sink));
  } else if (chunk_kib == 16) {
    const int64_t nb = (n16 + kTpb * 4 - 1) / (kTpb * 4);
    hipLaunchKernelGGL(read_chunk<4>, dim3(static_cast<unsigned>(nb)), dim3(kTpb), 0, s, p, n16,
                       static_cast<float *>(sink));
  } else {
    return static_cast<int>(hipErrorInvalidValue);
  }
  return static_cast<int>(hipGetLastError());
}

__attribute__((visibility("default"))) int ceiling_copy(const void *src, void *dst, size_t bytes, int chunk_kib,
                                                        hipStream_t s) {
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  if (!src || !dst || n16 < 1) return static_cast<int>(hipErrorInvalidValue);
  const f32x4 *p = static_cast<const f32x4 *>(src);
  f32x4 *q = static_cast<f32x4 *>(dst);
  if (chunk_kib == 64) {
    const int64_t nb = (n16 + kTpb * 16 - 1) / (kTpb * 16);
    hipLaunchKernelGGL(copy_chunk<16>, dim3(static_cast<unsigned>(nb)), dim3(kTpb), 0, s, p, q, n16);
  } else if (chunk_kib == 16) {
    const int64_t nb = (n16 + kTpb * 4 - 1) / (kTpb * 4);
    hipLaunchKernelGGL(copy_chunk<4>, dim3(static_cast<unsigned>(nb)), dim3(kTpb), 0, s, p, q, n16);
  } else {
    return static_cast<int>(hipErrorInvalidValue);
  }
  return static_cast<int>(hipGetLastError());
}

// src [1000][nchan] and dst [1001][nchan] FP64; nchan a multiple of C.
__attribute__((visibility("default"))) int ceiling_tile_rw(const double *src, double *dst, int64_t nchan, int C,
                                                           hipStream_t s) {
  if (!src || !dst || nchan < 1 || (C != 8 && C != 16) || nchan % C) return static_cast<int>(hipErrorInvalidValue);
  const unsigned nb = static_cast<unsigned>(nchan / C);
  if (C == 8)
    hipLaunchKernelGGL((tile_rw<8, 1000>), dim3(nb), dim3(1024), 0, s, src, dst, nchan);
  else
    hipLaunchKernelGGL((tile_rw<16, 1000>), dim3(nb), dim3(1024), 0, s, src, dst, nchan);
  return static_cast<int>(hipGetLastError());
}

}  // extern "C"
