// The library's static device scratch: one fixed array per GPU that the
// allocation-free apply (fftmv_apply_scratch) uses for the intermediate
// spectra and partial sums of an apply, in place of the plan's workspace.
// It exists for callers that cannot allocate device memory (code under
// stream capture, serving loops, harnesses that forbid allocation).
#include <hip/hip_runtime.h>

#include <mutex>

#include "common.hpp"
#include "internal.hpp"

namespace fftmv {

// Module-scope device array. In host code its name is a host-side stand-in,
// not a device address: host code only ever uses the address that
// hipGetSymbolAddress reports for the current device (scratch_device_ptr).
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxScratchDevices] = {};

// Zero `words` 4-byte words at base + r * pitch + off for r < rows (the pad
// columns of a row-major buffer).
__global__ __launch_bounds__(kBlock) void zero_cols_kernel(unsigned char *base, int64_t rows, int64_t pitch,
                                                           int64_t off, int64_t words) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (i >= rows * words) return;
  const int64_t r = i / words, w = i - r * words;
  *reinterpret_cast<uint32_t *>(base + r * pitch + off + 4 * w) = 0u;
}

}  // namespace

hipError_t scratch_device_ptr(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    // the address of this device's copy, looked up once with the device current
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return e;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_zero_cols(void *base, int64_t rows, int64_t pitch_bytes, int64_t off_bytes, int64_t bytes,
                            hipStream_t s) {
  if (rows <= 0 || bytes <= 0) return hipSuccess;
  if ((pitch_bytes | off_bytes | bytes) & 3) return hipErrorInvalidValue;
  const int64_t words = bytes / 4, n = rows * words;
  const int64_t nblocks = (n + kBlock - 1) / kBlock;
  if (!grid_fits(nblocks, kBlock)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(zero_cols_kernel, dim3(static_cast<unsigned>(nblocks)), dim3(kBlock), 0, s,
                     static_cast<unsigned char *>(base), rows, pitch_bytes, off_bytes, words);
  return hipGetLastError();
}

}  // namespace fftmv
