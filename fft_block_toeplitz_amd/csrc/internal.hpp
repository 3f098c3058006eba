// Host-side interface between the plan code and the kernel launchers.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace fftmv {

constexpr int kMaxPasses = 24;
constexpr int kMaxLds = 65536;      // bytes of LDS a 256-thread FFT workgroup may use
constexpr int kBlockWide = 1024;    // threads of a wide FFT workgroup
constexpr int kMaxLdsWide = 81920;  // LDS of a wide FFT workgroup: two fit a CU's 160 KiB
constexpr int kMaxChannelsPerBlock = 32;

// A dispatch carries its grid as a 32-bit count of work-items: a launch of
// nblocks workgroups of tpb threads fits when nblocks * tpb < 2^32.
// Launchers return hipErrorInvalidConfiguration for larger grids.
inline bool grid_fits(int64_t nblocks, int64_t tpb) {
  return nblocks >= 0 && tpb > 0 && nblocks <= static_cast<int64_t>(UINT32_MAX) / tpb;
}

// Stockham radix schedule of the length-L complex FFT that carries the
// length-2L real FFT (even samples in the real part, odd in the imaginary).
struct FftGeom {
  int L = 0;        // complex length (= Nt); 0 = unsupported length
  int npass = 0;
  int radix[kMaxPasses] = {};
  int ns[kMaxPasses] = {};      // product of the radices before this pass
  int twstep[kMaxPasses] = {};  // 2L / (ns * radix): exponent step in the w_{2L} table
};

// Radix schedule for L = 2^a 3^b 5^c 7^d: radix 8 while more than four
// factors of two remain, then 4 4 / 8 / 4 / 2, then the threes, fives and
// sevens. Usable on the host and, as a constant expression, in kernels
// specialised for one length.
constexpr FftGeom make_geometry(int L) {
  FftGeom g{};
  if (L < 1) return g;
  int r = L, a = 0, b3 = 0, b = 0, b7 = 0;
  while (r % 2 == 0) r /= 2, ++a;
  while (r % 3 == 0) r /= 3, ++b3;
  while (r % 5 == 0) r /= 5, ++b;
  while (r % 7 == 0) r /= 7, ++b7;
  if (r != 1 || a / 3 + 2 + b3 + b + b7 > kMaxPasses) return g;
  int np = 0;
  while (a > 4) {
    g.radix[np++] = 8;
    a -= 3;
  }
  if (a == 4) {
    g.radix[np++] = 4;
    g.radix[np++] = 4;
  } else if (a == 3) {
    g.radix[np++] = 8;
  } else if (a == 2) {
    g.radix[np++] = 4;
  } else if (a == 1) {
    g.radix[np++] = 2;
  }
  for (int i = 0; i < b3; ++i) g.radix[np++] = 3;
  for (int i = 0; i < b; ++i) g.radix[np++] = 5;
  for (int i = 0; i < b7; ++i) g.radix[np++] = 7;
  g.L = L;
  g.npass = np;
  int ns = 1;
  for (int p = 0; p < np; ++p) {
    g.ns[p] = ns;
    g.twstep[p] = 2 * L / (ns * g.radix[p]);
    ns *= g.radix[p];
  }
  return g;
}

// Bluestein (chirp-z) form of the length-L complex FFT for lengths without
// a radix schedule: with c[m] = exp(-pi i m^2 / L) = w_{2L}^(m^2 mod 2L),
//   Z[k] = c[k] sum_n (z[n] c[n]) conj(c[k - n])     (forward)
//   z[n] = conj(c[n]) sum_k (Z[k] conj(c[k])) c[n - k]   (inverse)
// each sum a circular convolution of length M (a power of two >= 2L - 1)
// done as M-point FFT, product with the filter's transform, inverse
// M-point FFT. Tables in both precisions (pointers to float or double
// complex).
struct BlueTables {
  FftGeom gM;                                   // radix schedule of M
  const void *tw32 = nullptr, *tw64 = nullptr;  // w_{2M}^t, t < 2M
  const void *hf32 = nullptr, *hf64 = nullptr;  // transform of conj(c), wrapped, / M (forward)
  const void *hi32 = nullptr, *hi64 = nullptr;  // transform of c, wrapped, / M (inverse)
};
// Smallest power of two >= 2L - 1 when L has no radix schedule (0 if L has
// one, or if the M-point tile would not fit a workgroup).
int64_t bluestein_length(int64_t L);

// Batched forward real FFT: nchan channels of Nt real samples (implicitly
// zero-padded to 2 Nt), channel ch at src[t * src_ld + ch]; writes the Nt+1
// bins of channel ch at dst + k * fstride + (ch / cpr) * ldr + ch % cpr, in
// complex64 (dst32) and/or complex128 (dst64).
struct FwdFftArgs {
  int64_t Nt = 0, nchan = 0;
  const void *src = nullptr;
  int64_t src_ld = 0;
  bool src_f32 = false;     // source holds float (else double)
  bool round_f32 = false;   // round double samples to binary32 before use
  void *dst32 = nullptr, *dst64 = nullptr;
  int64_t fstride32 = 0, ldr32 = 0, fstride64 = 0, ldr64 = 0, cpr = 1;
};

// Batched inverse real FFT + unpad: bins k = 0..Nt of channel ch at
// src[k * src_ld + ch] (complex); writes time steps 0..Nt-1 at
// dst[t * dst_ld + ch] as float (dst_f32) or double.
struct InvFftArgs {
  int64_t Nt = 0, nchan = 0;
  const void *src = nullptr;
  int64_t src_ld = 0;
  bool src_f32 = false;
  void *dst = nullptr;
  int64_t dst_ld = 0;
  bool dst_f32 = false;
  bool round_f32 = false;  // round to binary32 before a double store
};

// Per-frequency complex GEMV over Fhat [K][Nd][ldF].
struct SbgemvArgs {
  int64_t K = 0, Nd = 0, Nm = 0;
  const void *F = nullptr;  // complex64 or complex128, per compute precision
  int64_t ldF = 0;          // complex elements per row (even for complex64)
  const void *x = nullptr;  // input  [K][ldx] complex (float if x_f32)
  int64_t ldx = 0;
  bool x_f32 = false;
  void *y = nullptr;        // output [K][ldy] complex (float if y_f32)
  int64_t ldy = 0;
  bool y_f32 = false;
  // workspace for partial sums (F* tall blocks and row segments, F column
  // chunks), part_bytes long; null keeps the one-pass kernels
  void *part = nullptr;
  size_t part_bytes = 0;
};

// Real [rows][cols] copy with precision change: dst[r*ldd+c] = src[r*lds+c].
struct CastArgs {
  int64_t rows = 0, cols = 0;
  const void *src = nullptr;
  int64_t lds = 0;
  bool src_f32 = false;
  void *dst = nullptr;
  int64_t ldd = 0;
  bool dst_f32 = false;
};

// FFT launch shape: C channels per workgroup (power of two), the
// per-thread register budget VMAX (complex values held during a pass) and
// the workgroup size (kBlock or kBlockWide threads).
struct FftLaunch {
  int C = 0;
  int vmax = 0;
  int tpb = 0;
};
FftLaunch fft_launch_config(const FftGeom &g, bool f32, int64_t nchan);
// Channels per FFT workgroup for this schedule, precision and batch size; 0
// if the transform does not fit.
int fft_channels_per_block(const FftGeom &g, bool f32, int64_t nchan);

// blue: Bluestein tables when the length has no radix schedule, else null
hipError_t launch_fft_forward(const FftGeom &g, const FwdFftArgs &a, bool compute_f32, const void *tw,
                              hipStream_t s, const BlueTables *blue = nullptr);
hipError_t launch_fft_inverse(const FftGeom &g, const InvFftArgs &a, bool compute_f32, const void *tw,
                              hipStream_t s, const BlueTables *blue = nullptr);
// Fixed-length kernels (fft_fixed_fwd.hip, fft_fixed_inv.hip): launch and return true when one
// covers this transform (*err: an error found before the launch), else return false and launch
// nothing.
bool launch_fft_forward_fixed(const FftGeom &g, const FwdFftArgs &a, bool compute_f32, const void *tw, hipStream_t s,
                              hipError_t *err);
// The setup transform of a wide batch (fft_setup.hip): Nt = L = 1000 or 2000, FP64 samples,
// frequency blocks of cpr-channel rows; tw = w_2L^t, t < 2L, complex128.
hipError_t launch_fft_setup_wide(int L, const FwdFftArgs &a, const void *tw, hipStream_t s);
bool launch_fft_inverse_fixed(const FftGeom &g, const InvFftArgs &a, bool compute_f32, const void *tw,
                              hipStream_t s);
hipError_t launch_sbgemv_n(const SbgemvArgs &a, bool compute_f32, hipStream_t s);
hipError_t launch_sbgemv_c(const SbgemvArgs &a, bool compute_f32, hipStream_t s);
// Bytes of the GEMV workspace for this shape: partial sums of the F*
// tall-block form and row segments, and of the F column chunks (the largest
// over both directions and compute precisions); 0 when no launch needs it.
size_t sbgemv_part_bytes(int64_t K, int64_t Nd, int64_t Nm);
hipError_t launch_cast(const CastArgs &a, hipStream_t s);

// The static device scratch of the allocation-free apply (scratch.hip):
// kScratchBytes per GPU, 256-byte aligned. scratch_device_ptr returns the
// current device's copy (its address looked up once per device).
constexpr size_t kScratchBytes = size_t(128) << 20;
hipError_t scratch_device_ptr(void **out);
// Zero `bytes` bytes (a multiple of 4) at base + r * pitch_bytes + off_bytes
// for every row r < rows, with a kernel (no memset node in a captured graph).
hipError_t launch_zero_cols(void *base, int64_t rows, int64_t pitch_bytes, int64_t off_bytes, int64_t bytes,
                            hipStream_t s);

// Lanczos process on the per-frequency Gram matrices (condition.hip). One
// frequency's vectors have n complex entries; vector j of frequency k is
// Q + (j * K + k) * ldq (complex128).
constexpr int kMaxLanczos = 512;
struct LanczosArgs {
  int64_t K = 0, n = 0;
  double *Q = nullptr;  // basis [J+1][K][ldq] complex128
  int64_t ldq = 0;
  double *z = nullptr;  // G q_j on entry to a step [K][ldz] complex128
  int64_t ldz = 0;
  void *xin = nullptr;  // the next GEMV input [K][ldx], complex64 if x_f32
  int64_t ldx = 0;
  bool x_f32 = false;
  double *alpha = nullptr, *beta = nullptr;  // [J][K]
  int *len = nullptr;                        // [K] completed steps (negative once stopped)
};
hipError_t launch_lanczos_start(const LanczosArgs &a, hipStream_t s);
hipError_t launch_lanczos_step(const LanczosArgs &a, int j, hipStream_t s);
// sigma[2k] = largest, sigma[2k+1] = smallest singular value of block k
hipError_t launch_lanczos_extremes(const LanczosArgs &a, double *sigma, hipStream_t s);

}  // namespace fftmv
