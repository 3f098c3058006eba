// Host side of the fftmv C ABI: plan construction, precision-mask dispatch
// and the launch sequence of the five stages of "Mixed-precision FFTMatvec
// performance optimization on AMD GPUs", section 1.1 (sections 1.2 and 2.2
// for the adjoint and the per-stage precision choice).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <complex>
#include <cstdint>
#include <cstring>
#include <new>

#include "fftmv.h"
#include "internal.hpp"

using namespace fftmv;

namespace {

constexpr int kVersion = (0 << 16) | (1 << 8) | 0;

// Buffers between stages: stage s of direction dir writes buf[dir][s].
struct StageBuf {
  void *p = nullptr;
  int64_t ld = 0;  // elements per row
};

}  // namespace

struct fftmv_plan_s {
  int device = 0;
  int64_t Nm = 0, Nd = 0, Nt = 0, K = 0;
  uint32_t prec = 0, flags = 0;
  FftGeom geom;
  bool blue = false;  // Bluestein form (Nt without a radix schedule)
  BlueTables bt;
  void *fhat32 = nullptr, *fhat64 = nullptr;
  int64_t ldF32 = 0, ldF64 = 0;
  void *tw32 = nullptr, *tw64 = nullptr;
  StageBuf buf[2][5];
  void *part = nullptr;  // GEMV partial sums (F* tall blocks / row segments, F column chunks)
  size_t part_bytes = 0;
  size_t fhat_bytes = 0, ws_bytes = 0;
  void *allocs[16] = {};
  int nalloc = 0;
};

namespace {

bool fp32(uint32_t prec, int dir, int stage) { return (prec >> (5 * dir + stage - 1)) & 1u; }

// Leading dimension of rows of n entries: even, so that 16-byte vectors of
// two complex64 entries never straddle rows; and for long rows (n >= 1024,
// at most 3% of padding) a multiple of 32 entries, so that every row starts
// on a 256-byte boundary (complex64) -- a wave's 1 KiB load then never
// shares a cache line with the previous row. Measured on the frequency
// blocks at Nm = 5000 (rows of 40000 bytes otherwise, every other one half a
// line off): the plain SBGEMV reads ~4% fewer bytes and runs faster.
int64_t padded_ld(int64_t n) {
  if (n >= 1024) return (n + 31) & ~int64_t(31);
  return (n + 1) & ~int64_t(1);
}

// Largest Nm: a row of Nm complex128 entries spans at most 2 GiB, so the
// GEMV kernels' 32-bit in-row byte offsets and row buffer descriptors
// cover it.
constexpr int64_t kMaxNm = int64_t(1) << 27;

bool mul_ok(int64_t a, int64_t b, int64_t *out) { return !__builtin_mul_overflow(a, b, out); }

int status_from_hip(hipError_t e) {
  if (e == hipSuccess) return FFTMV_SUCCESS;
  if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation) return FFTMV_ERR_OUT_OF_MEMORY;
  if (e == hipErrorInvalidConfiguration) return FFTMV_ERR_UNSUPPORTED_SIZE;  // a grid above 2^32 work-items
  return FFTMV_ERR_HIP;
}

#define FFTMV_TRY(expr)                              \
  do {                                               \
    hipError_t e_ = (expr);                          \
    if (e_ != hipSuccess) return status_from_hip(e_); \
  } while (0)

bool build_geometry(int64_t L, FftGeom *g) {
  // lengths with more than kMaxPasses passes are far above the LDS limit
  if (L < 1 || L > (int64_t(1) << 20)) return false;
  *g = make_geometry(static_cast<int>(L));
  return g->L == L;
}

// exp(-2 pi i t / N) with the angle reduced exactly in integers to
// [0, pi/4] by the symmetries of sine and cosine, so that multiples of pi/4
// come out exact (or correctly rounded) and the table is symmetric.
void unit_root(int64_t t, int64_t N, double *re, double *im) {
  int64_t u = 4 * (t % N);  // angle = 2 pi u / (4N)
  const int64_t full = 4 * N;
  double ss = 1.0, sc = 1.0;
  if (u > full / 2) {  // 2 pi - a
    u = full - u;
    ss = -1.0;
  }
  if (u > N) {  // pi - a
    u = 2 * N - u;
    sc = -1.0;
  }
  bool swap = false;
  if (2 * u > N) {  // pi/2 - a
    u = N - u;
    swap = true;
  }
  const double a = (M_PI / 2.0) * static_cast<double>(u) / static_cast<double>(N);
  double c = std::cos(a), s = std::sin(a);
  if (u == 0) c = 1.0, s = 0.0;
  if (swap) std::swap(c, s);
  *re = sc * c;
  *im = -(ss * s);
}

// In-place length-n FFT (n a power of two, exponent sign -1) in long
// double, for the Bluestein filter tables.
void host_fft(std::complex<long double> *x, int64_t n) {
  for (int64_t i = 1, j = 0; i < n; ++i) {  // bit-reversal permutation
    int64_t bit = n >> 1;
    for (; j & bit; bit >>= 1) j ^= bit;
    j ^= bit;
    if (i < j) std::swap(x[i], x[j]);
  }
  const long double pi = 3.141592653589793238462643383279502884L;
  for (int64_t len = 2; len <= n; len <<= 1) {
    for (int64_t k = 0; k < len / 2; ++k) {
      const long double ang = -2.0L * pi * static_cast<long double>(k) / static_cast<long double>(len);
      const std::complex<long double> w(std::cos(ang), std::sin(ang));
      for (int64_t i = 0; i < n; i += len) {
        const std::complex<long double> u = x[i + k], v = x[i + k + len / 2] * w;
        x[i + k] = u + v;
        x[i + k + len / 2] = u - v;
      }
    }
  }
}

void release(fftmv_plan_s *p) {
  for (int i = 0; i < p->nalloc; ++i) (void)hipFree(p->allocs[i]);
  p->nalloc = 0;
}

hipError_t dev_alloc(fftmv_plan_s *p, void **ptr, size_t bytes) {
  if (p->nalloc >= 16) return hipErrorUnknown;
  void *q = nullptr;
  hipError_t e = hipMalloc(&q, bytes ? bytes : 16);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return e;
  }
  p->allocs[p->nalloc++] = q;
  *ptr = q;
  return hipSuccess;
}

bool aligned8(const void *q) { return (reinterpret_cast<uintptr_t>(q) & 7u) == 0; }

struct cx64 {
  double re, im;
};
struct cx32 {
  float re, im;
};

// stage-boundary buffer precisions: the narrower of the two stages
bool buf_f32(uint32_t prec, int dir, int s) { return fp32(prec, dir, s) || fp32(prec, dir, s + 1); }

int64_t channels_in(const fftmv_plan_s *p, int dir) { return dir == 0 ? p->Nm : p->Nd; }
int64_t channels_out(const fftmv_plan_s *p, int dir) { return dir == 0 ? p->Nd : p->Nm; }

bool needs_fhat32(uint32_t prec) { return fp32(prec, 0, 3) || fp32(prec, 1, 3); }
bool needs_fhat64(uint32_t prec) { return !fp32(prec, 0, 3) || !fp32(prec, 1, 3); }

const void *twiddles(const fftmv_plan_s *p, bool f32) { return f32 ? p->tw32 : p->tw64; }

// ------------------------------------------------------------- stages
// Stage 1 alone: m (FP64) -> buf 1 (the live half of the padded input).
hipError_t stage_pad(const fftmv_plan_s *p, int dir, const double *in, hipStream_t s) {
  CastArgs a;
  a.rows = p->Nt;
  a.cols = channels_in(p, dir);
  a.src = in;
  a.lds = a.cols;
  a.src_f32 = false;
  a.dst = p->buf[dir][1].p;
  a.ldd = p->buf[dir][1].ld;
  a.dst_f32 = buf_f32(p->prec, dir, 1);
  return launch_cast(a, s);
}

// Stage 2: forward FFT of the input channels into buf 2. With from_user the
// stage-1 pad is folded into the load (reads the FP64 input directly and
// rounds it when stage 1 or 2 is FP32).
hipError_t stage_fft(const fftmv_plan_s *p, int dir, const double *user_in, bool from_user, hipStream_t s) {
  const bool cf32 = fp32(p->prec, dir, 2);
  FwdFftArgs a;
  a.Nt = p->Nt;
  a.nchan = channels_in(p, dir);
  if (from_user) {
    a.src = user_in;
    a.src_ld = a.nchan;
    a.src_f32 = false;
    a.round_f32 = fp32(p->prec, dir, 1);
  } else {
    a.src = p->buf[dir][1].p;
    a.src_ld = p->buf[dir][1].ld;
    a.src_f32 = buf_f32(p->prec, dir, 1);
    a.round_f32 = false;
  }
  const StageBuf &o = p->buf[dir][2];
  if (buf_f32(p->prec, dir, 2)) {
    a.dst32 = o.p;
    a.fstride32 = o.ld;
    a.ldr32 = 0;
  } else {
    a.dst64 = o.p;
    a.fstride64 = o.ld;
    a.ldr64 = 0;
  }
  a.cpr = a.nchan;
  return launch_fft_forward(p->geom, a, cf32, twiddles(p, cf32), s, p->blue ? &p->bt : nullptr);
}

// Stage 3: per-frequency GEMV (F) or conjugate-transpose GEMV (F*).
hipError_t stage_sbgemv(const fftmv_plan_s *p, int dir, hipStream_t s) {
  const bool cf32 = fp32(p->prec, dir, 3);
  SbgemvArgs a;
  a.K = p->K;
  a.Nd = p->Nd;
  a.Nm = p->Nm;
  a.F = cf32 ? p->fhat32 : p->fhat64;
  a.ldF = cf32 ? p->ldF32 : p->ldF64;
  a.x = p->buf[dir][2].p;
  a.ldx = p->buf[dir][2].ld;
  a.x_f32 = buf_f32(p->prec, dir, 2);
  a.y = p->buf[dir][3].p;
  a.ldy = p->buf[dir][3].ld;
  a.y_f32 = buf_f32(p->prec, dir, 3);
  a.part = p->part;
  a.part_bytes = p->part_bytes;
  if (!a.F) return hipErrorInvalidValue;
  return dir == 0 ? launch_sbgemv_n(a, cf32, s) : launch_sbgemv_c(a, cf32, s);
}

// Stage 4: inverse FFT of the output channels. With to_user the stage-5
// unpad is folded into the store (writes FP64, rounded when stage 5 is FP32).
hipError_t stage_ifft(const fftmv_plan_s *p, int dir, double *user_out, bool to_user, hipStream_t s) {
  const bool cf32 = fp32(p->prec, dir, 4);
  InvFftArgs a;
  a.Nt = p->Nt;
  a.nchan = channels_out(p, dir);
  a.src = p->buf[dir][3].p;
  a.src_ld = p->buf[dir][3].ld;
  a.src_f32 = buf_f32(p->prec, dir, 3);
  if (to_user) {
    a.dst = user_out;
    a.dst_ld = a.nchan;
    a.dst_f32 = false;
    a.round_f32 = fp32(p->prec, dir, 5);
  } else {
    a.dst = p->buf[dir][4].p;
    a.dst_ld = p->buf[dir][4].ld;
    a.dst_f32 = buf_f32(p->prec, dir, 4);
    a.round_f32 = false;
  }
  return launch_fft_inverse(p->geom, a, cf32, twiddles(p, cf32), s, p->blue ? &p->bt : nullptr);
}

// Stage 5 alone: buf 4 -> FP64 output.
hipError_t stage_unpad(const fftmv_plan_s *p, int dir, double *out, hipStream_t s) {
  CastArgs a;
  a.rows = p->Nt;
  a.cols = channels_out(p, dir);
  a.src = p->buf[dir][4].p;
  a.lds = p->buf[dir][4].ld;
  a.src_f32 = buf_f32(p->prec, dir, 4);
  a.dst = out;
  a.ldd = a.cols;
  a.dst_f32 = false;
  return launch_cast(a, s);
}

hipError_t run_range(const fftmv_plan_s *p, int dir, int first, int last, const double *in, double *out,
                     hipStream_t s) {
  hipError_t e = hipSuccess;
  for (int st = first; st <= last && e == hipSuccess; ++st) {
    switch (st) {
      case 1: e = stage_pad(p, dir, in, s); break;
      case 2: e = stage_fft(p, dir, nullptr, false, s); break;
      case 3: e = stage_sbgemv(p, dir, s); break;
      case 4: e = stage_ifft(p, dir, nullptr, false, s); break;
      default: e = stage_unpad(p, dir, out, s); break;
    }
  }
  return e;
}

// Work is launched on the current device: it must be the plan's.
bool on_plan_device(const fftmv_plan_s *p) {
  int d = -1;
  return hipGetDevice(&d) == hipSuccess && d == p->device;
}

// The FP64 input [Nt][n_in] and output [Nt][n_out] of one direction overlap.
bool overlap(const fftmv_plan_s *p, int dir, const double *in, const double *out) {
  const int64_t n_in = dir == FFTMV_DIR_F ? p->Nm : p->Nd, n_out = dir == FFTMV_DIR_F ? p->Nd : p->Nm;
  const uintptr_t i0 = reinterpret_cast<uintptr_t>(in), o0 = reinterpret_cast<uintptr_t>(out);
  const uintptr_t i1 = i0 + static_cast<uintptr_t>(p->Nt * n_in) * sizeof(double);
  const uintptr_t o1 = o0 + static_cast<uintptr_t>(p->Nt * n_out) * sizeof(double);
  return i0 < o1 && o0 < i1;
}

bool apply_args_ok(const fftmv_plan_s *p, int dir, const double *in, double *out) {
  if (!p || !in || !out || !aligned8(in) || !aligned8(out)) return false;
  return !overlap(p, dir, in, out) && on_plan_device(p);
}

// The launches of one apply (five-kernel or fused form) with p's buffers.
hipError_t launch_apply(const fftmv_plan_s *p, int dir, const double *in, double *out, hipStream_t s) {
  if (p->flags & FFTMV_FLAG_STAGED) return run_range(p, dir, 1, 5, in, out, s);
  hipError_t e = stage_fft(p, dir, in, true, s);
  if (e == hipSuccess) e = stage_sbgemv(p, dir, s);
  if (e == hipSuccess) e = stage_ifft(p, dir, out, true, s);
  return e;
}

int apply_dir(fftmv_plan_t p, int dir, const double *in, double *out, hipStream_t s) {
  if (!apply_args_ok(p, dir, in, out)) return FFTMV_ERR_INVALID_ARG;
  try {
    return status_from_hip(launch_apply(p, dir, in, out, s));
  } catch (...) {
    return FFTMV_ERR_INTERNAL;
  }
}

// Bytes of the static scratch an apply of direction dir takes, and the
// plan's stage buffers and GEMV workspace laid out in it (each region
// 256-byte aligned, buffers in the precision the mask gives them). Returns
// false when they do not fit kScratchBytes.
bool scratch_layout(const fftmv_plan_s *p, int dir, unsigned char *base, fftmv_plan_s *view, size_t *need) {
  const bool staged = p->flags & FFTMV_FLAG_STAGED;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += (bytes + 255) & ~size_t(255);
    return at;
  };
  for (int st = staged ? 1 : 2; st <= (staged ? 4 : 3); ++st) {
    const bool cplx = st == 2 || st == 3;
    const int64_t rows = cplx ? p->K : p->Nt;
    const size_t esz = (cplx ? 16 : 8) / (buf_f32(p->prec, dir, st) ? 2 : 1);
    const size_t at = take(static_cast<size_t>(rows * p->buf[dir][st].ld) * esz);
    if (view) view->buf[dir][st].p = base + at;
  }
  if (p->part_bytes) {
    const size_t at = take(p->part_bytes);
    if (view) view->part = base + at;
  }
  *need = off;
  return off <= kScratchBytes;
}

int setup_impl(fftmv_plan_s *p, const double *F, hipStream_t s) {
  const int64_t Nm = p->Nm, Nd = p->Nd, Nt = p->Nt, K = p->K;
  const bool want32 = needs_fhat32(p->prec) || (p->flags & FFTMV_FLAG_FHAT_BOTH);
  const bool want64 = needs_fhat64(p->prec) || (p->flags & FFTMV_FLAG_FHAT_BOTH);

  // Fhat
  int64_t n32 = 0, n64 = 0, tmp = 0;
  p->ldF32 = padded_ld(Nm);
  p->ldF64 = padded_ld(Nm);
  if (!mul_ok(K, Nd, &tmp) || !mul_ok(tmp, p->ldF32, &n32) || !mul_ok(tmp, p->ldF64, &n64) ||
      !mul_ok(n64, 16, &tmp))
    return FFTMV_ERR_OUT_OF_MEMORY;
  // the transform writes every (row, column < Nm) entry; only the padding
  // columns Nm..ld-1 of each of the K Nd rows are cleared here
  if (want32) {
    FFTMV_TRY(dev_alloc(p, &p->fhat32, static_cast<size_t>(n32) * 8));
    FFTMV_TRY(launch_zero_cols(p->fhat32, K * Nd, p->ldF32 * 8, Nm * 8, (p->ldF32 - Nm) * 8, s));
    p->fhat_bytes += static_cast<size_t>(n32) * 8;
  }
  if (want64) {
    FFTMV_TRY(dev_alloc(p, &p->fhat64, static_cast<size_t>(n64) * 16));
    FFTMV_TRY(launch_zero_cols(p->fhat64, K * Nd, p->ldF64 * 16, Nm * 16, (p->ldF64 - Nm) * 16, s));
    p->fhat_bytes += static_cast<size_t>(n64) * 16;
  }

  // twiddles: w_N^t for t < N = 2 Nt, in both precisions
  const int64_t N = 2 * Nt;
  {
    double *h64 = new (std::nothrow) double[2 * N];
    float *h32 = new (std::nothrow) float[2 * N];
    if (!h64 || !h32) {
      delete[] h64;
      delete[] h32;
      return FFTMV_ERR_INTERNAL;
    }
    for (int64_t t = 0; t < N; ++t) {
      unit_root(t, N, &h64[2 * t], &h64[2 * t + 1]);
      h32[2 * t] = static_cast<float>(h64[2 * t]);
      h32[2 * t + 1] = static_cast<float>(h64[2 * t + 1]);
    }
    hipError_t e = dev_alloc(p, &p->tw64, static_cast<size_t>(N) * 16);
    if (e == hipSuccess) e = dev_alloc(p, &p->tw32, static_cast<size_t>(N) * 8);
    if (e == hipSuccess) e = hipMemcpy(p->tw64, h64, static_cast<size_t>(N) * 16, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(p->tw32, h32, static_cast<size_t>(N) * 8, hipMemcpyHostToDevice);
    delete[] h64;
    delete[] h32;
    FFTMV_TRY(e);
    p->ws_bytes += static_cast<size_t>(N) * 24;
  }

  // Bluestein tables: w_{2M}^t, and the transforms (divided by M) of the
  // wrapped filters conj(c) (forward) and c (inverse), c[m] = w_{2L}^(m^2 mod 2L)
  if (p->blue) {
    const int64_t M = p->bt.gM.L, n64 = 4 * M;  // 2M twiddles + M + M filter values
    std::complex<long double> *h = new (std::nothrow) std::complex<long double>[M];
    double *t64 = new (std::nothrow) double[2 * n64];
    float *t32 = new (std::nothrow) float[2 * n64];
    if (!h || !t64 || !t32) {
      delete[] h;
      delete[] t64;
      delete[] t32;
      return FFTMV_ERR_INTERNAL;
    }
    for (int64_t t = 0; t < 2 * M; ++t) unit_root(t, 2 * M, &t64[2 * t], &t64[2 * t + 1]);
    for (int64_t m = 0; m < M; ++m) h[m] = 0.0L;
    for (int64_t m = 0; m < Nt; ++m) {
      double re, im;
      unit_root((m * m) % (2 * Nt), 2 * Nt, &re, &im);
      h[m] = std::complex<long double>(re, -im);  // conj(c[m])
      if (m > 0) h[M - m] = h[m];                  // c is even in m
    }
    host_fft(h, M);
    double *hf = t64 + 4 * M, *hi = t64 + 6 * M;
    for (int64_t k = 0; k < M; ++k) {
      const std::complex<long double> v = h[k] / static_cast<long double>(M);
      const std::complex<long double> w = std::conj(h[(M - k) % M]) / static_cast<long double>(M);
      hf[2 * k] = static_cast<double>(v.real());
      hf[2 * k + 1] = static_cast<double>(v.imag());
      hi[2 * k] = static_cast<double>(w.real());
      hi[2 * k + 1] = static_cast<double>(w.imag());
    }
    for (int64_t i = 0; i < 2 * n64; ++i) t32[i] = static_cast<float>(t64[i]);
    void *tab = nullptr;
    hipError_t e = dev_alloc(p, &tab, static_cast<size_t>(n64) * 24);
    if (e == hipSuccess) e = hipMemcpy(tab, t64, static_cast<size_t>(n64) * 16, hipMemcpyHostToDevice);
    if (e == hipSuccess)
      e = hipMemcpy(static_cast<char *>(tab) + n64 * 16, t32, static_cast<size_t>(n64) * 8, hipMemcpyHostToDevice);
    delete[] h;
    delete[] t64;
    delete[] t32;
    FFTMV_TRY(e);
    const cx64 *d64 = static_cast<const cx64 *>(tab);
    const cx32 *d32 = reinterpret_cast<const cx32 *>(static_cast<const char *>(tab) + n64 * 16);
    p->bt.tw64 = d64;
    p->bt.hf64 = d64 + 2 * M;
    p->bt.hi64 = d64 + 3 * M;
    p->bt.tw32 = d32;
    p->bt.hf32 = d32 + 2 * M;
    p->bt.hi32 = d32 + 3 * M;
    p->ws_bytes += static_cast<size_t>(n64) * 24;
  }

  // stage buffers, sized for FP64 so that any precision mask fits
  for (int dir = 0; dir < 2; ++dir) {
    const int64_t ldi = padded_ld(channels_in(p, dir)), ldo = padded_ld(channels_out(p, dir));
    const int64_t rows[5] = {0, Nt, K, K, Nt};
    const int64_t lds[5] = {0, ldi, ldi, ldo, ldo};
    const int64_t esz[5] = {0, 8, 16, 16, 8};
    for (int st = 1; st <= 4; ++st) {
      int64_t n = 0, bytes = 0;
      if (!mul_ok(rows[st], lds[st], &n) || !mul_ok(n, esz[st], &bytes)) return FFTMV_ERR_OUT_OF_MEMORY;
      FFTMV_TRY(dev_alloc(p, &p->buf[dir][st].p, static_cast<size_t>(bytes)));
      FFTMV_TRY(hipMemsetAsync(p->buf[dir][st].p, 0, static_cast<size_t>(bytes), s));
      p->buf[dir][st].ld = lds[st];
      p->ws_bytes += static_cast<size_t>(bytes);
    }
  }

  // partial sums of the GEMV forms that split a frequency's work (F*: tall
  // blocks and row segments; F: column chunks), for either precision
  p->part_bytes = sbgemv_part_bytes(K, Nd, Nm);
  if (p->part_bytes) {
    FFTMV_TRY(dev_alloc(p, &p->part, p->part_bytes));
    p->ws_bytes += p->part_bytes;
  }

  // Fhat_k = DFT of every zero-padded (r, c) series, computed in FP64 and
  // rounded once to each stored precision
  FwdFftArgs a;
  a.Nt = Nt;
  a.nchan = Nd * Nm;
  a.src = F;
  a.src_ld = Nd * Nm;
  a.src_f32 = false;
  a.round_f32 = false;
  a.dst32 = p->fhat32;
  a.fstride32 = Nd * p->ldF32;
  a.ldr32 = p->ldF32;
  a.dst64 = p->fhat64;
  a.fstride64 = Nd * p->ldF64;
  a.ldr64 = p->ldF64;
  a.cpr = Nm;
  FFTMV_TRY(launch_fft_forward(p->geom, a, false, p->tw64, s, p->blue ? &p->bt : nullptr));
  FFTMV_TRY(hipStreamSynchronize(s));
  return FFTMV_SUCCESS;
}

// Device memory of one condition estimate, freed on every return path.
struct TempAllocs {
  hipStream_t stream = nullptr;
  void *p[8] = {};
  int n = 0;
  hipError_t get(void **out, size_t bytes) {
    void *q = nullptr;
    hipError_t e = hipMalloc(&q, bytes ? bytes : 16);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return e;
    }
    p[n++] = q;
    *out = q;
    return hipSuccess;
  }
  ~TempAllocs() {
    (void)hipStreamSynchronize(stream);  // nothing queued may still use them
    for (int i = 0; i < n; ++i) (void)hipFree(p[i]);
  }
};

// Lanczos on the smaller Gram matrix of every Fhat_k: when Nd <= Nm,
// G_k = Fhat_k Fhat_k^H (conjugate-transpose product, then the plain one),
// else G_k = Fhat_k^H Fhat_k (the other order).
int condition_impl(fftmv_plan_s *p, int iters, double *kappa, double *smax, double *smin, hipStream_t s) {
  const int64_t K = p->K, Nm = p->Nm, Nd = p->Nd;
  const bool wide = Nd <= Nm;
  const int64_t n = wide ? Nd : Nm, nlong = wide ? Nm : Nd;
  int64_t J = iters > 0 ? iters : std::min<int64_t>(n, 128);
  J = std::min<int64_t>(std::min<int64_t>(J, n), kMaxLanczos);
  const bool f32 = p->fhat64 == nullptr;  // use the complex128 copy when there is one
  const int64_t ldq = padded_ld(n), ldl = padded_ld(nlong);
  const size_t csz = f32 ? 8 : 16;

  TempAllocs t;
  t.stream = s;
  LanczosArgs a;
  a.K = K;
  a.n = n;
  a.ldq = ldq;
  a.ldz = ldq;
  a.ldx = ldq;
  a.x_f32 = f32;
  void *Q = nullptr, *z = nullptr, *xin = nullptr, *y = nullptr, *al = nullptr, *be = nullptr, *len = nullptr,
       *sig = nullptr;
  const size_t vec = static_cast<size_t>(K * ldq);
  FFTMV_TRY(t.get(&Q, static_cast<size_t>(J + 1) * vec * 16));
  FFTMV_TRY(t.get(&z, vec * 16));
  FFTMV_TRY(t.get(&xin, vec * csz));
  FFTMV_TRY(t.get(&y, static_cast<size_t>(K * ldl) * csz));
  FFTMV_TRY(t.get(&al, static_cast<size_t>(J * K) * 8));
  FFTMV_TRY(t.get(&be, static_cast<size_t>(J * K) * 8));
  FFTMV_TRY(t.get(&len, static_cast<size_t>(K) * 4));
  FFTMV_TRY(t.get(&sig, static_cast<size_t>(K) * 16));
  // the GEMVs read whole 16-byte vectors: padding entries must hold zeros
  FFTMV_TRY(hipMemsetAsync(xin, 0, vec * csz, s));
  FFTMV_TRY(hipMemsetAsync(y, 0, static_cast<size_t>(K * ldl) * csz, s));
  a.Q = static_cast<double *>(Q);
  a.z = static_cast<double *>(z);
  a.xin = xin;
  a.alpha = static_cast<double *>(al);
  a.beta = static_cast<double *>(be);
  a.len = static_cast<int *>(len);

  SbgemvArgs g1, g2;
  g1.K = g2.K = K;
  g1.Nd = g2.Nd = Nd;
  g1.Nm = g2.Nm = Nm;
  g1.F = g2.F = f32 ? p->fhat32 : p->fhat64;
  g1.ldF = g2.ldF = f32 ? p->ldF32 : p->ldF64;
  // the plan's GEMV workspace (sized for this shape; the estimate is ordered
  // with the plan's applies), so that tall or few-frequency blocks take the
  // split forms here too
  g1.part = g2.part = p->part;
  g1.part_bytes = g2.part_bytes = p->part_bytes;
  g1.x = xin;
  g1.ldx = ldq;
  g1.x_f32 = f32;
  g1.y = y;
  g1.ldy = ldl;
  g1.y_f32 = f32;
  g2.x = y;
  g2.ldx = ldl;
  g2.x_f32 = f32;
  g2.y = z;
  g2.ldy = ldq;
  g2.y_f32 = false;

  FFTMV_TRY(launch_lanczos_start(a, s));
  for (int j = 0; j < J; ++j) {
    if (wide) {
      FFTMV_TRY(launch_sbgemv_c(g1, f32, s));
      FFTMV_TRY(launch_sbgemv_n(g2, f32, s));
    } else {
      FFTMV_TRY(launch_sbgemv_n(g1, f32, s));
      FFTMV_TRY(launch_sbgemv_c(g2, f32, s));
    }
    FFTMV_TRY(launch_lanczos_step(a, j, s));
  }
  FFTMV_TRY(launch_lanczos_extremes(a, static_cast<double *>(sig), s));
  double *h = new (std::nothrow) double[2 * K];
  if (!h) return FFTMV_ERR_INTERNAL;
  hipError_t e = hipMemcpyAsync(h, sig, static_cast<size_t>(K) * 16, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    delete[] h;
    return status_from_hip(e);
  }
  double hi = 0.0, lo = INFINITY;
  for (int64_t k = 0; k < K; ++k) {
    hi = std::max(hi, h[2 * k]);
    lo = std::min(lo, h[2 * k + 1]);
    if (smax) smax[k] = h[2 * k];
    if (smin) smin[k] = h[2 * k + 1];
  }
  delete[] h;
  if (kappa) *kappa = lo > 0.0 ? hi / lo : INFINITY;
  return FFTMV_SUCCESS;
}

}  // namespace

extern "C" {

int fftmv_setup(fftmv_plan_t *out, const double *F_dev, int64_t Nm, int64_t Nd, int64_t Nt, uint32_t mask,
                hipStream_t stream) {
  if (!out || !F_dev || !aligned8(F_dev) || Nm < 1 || Nd < 1 || Nt < 1) return FFTMV_ERR_INVALID_ARG;
  if (mask & ~(FFTMV_PREC_BITS | FFTMV_FLAG_BITS)) return FFTMV_ERR_INVALID_ARG;
  if (Nm > INT32_MAX || Nd > INT32_MAX) return FFTMV_ERR_UNSUPPORTED_SIZE;
  // the GEMV kernels address a row of Fhat with 32-bit byte offsets
  if (Nm > kMaxNm) return FFTMV_ERR_UNSUPPORTED_SIZE;
  if (Nt > 4096) return FFTMV_ERR_UNSUPPORTED_SIZE;
  try {
    fftmv_plan_s *p = new (std::nothrow) fftmv_plan_s();
    if (!p) return FFTMV_ERR_INTERNAL;
    p->Nm = Nm;
    p->Nd = Nd;
    p->Nt = Nt;
    p->K = Nt + 1;
    p->prec = mask & FFTMV_PREC_BITS;
    p->flags = mask & FFTMV_FLAG_BITS;
    const bool radix = build_geometry(Nt, &p->geom) && fft_channels_per_block(p->geom, false, 1) > 0 &&
                       fft_channels_per_block(p->geom, true, 1) > 0;
    if (!radix) {
      // lengths without a radix schedule: Bluestein form over M points
      const int64_t M = bluestein_length(Nt);
      if (M == 0) {
        delete p;
        return FFTMV_ERR_UNSUPPORTED_SIZE;
      }
      p->blue = true;
      p->bt.gM = make_geometry(static_cast<int>(M));
      p->geom = FftGeom{};
      p->geom.L = static_cast<int>(Nt);
    }
    if (hipGetDevice(&p->device) != hipSuccess) {
      delete p;
      return FFTMV_ERR_HIP;
    }
    int st = setup_impl(p, F_dev, stream);
    if (st != FFTMV_SUCCESS) {
      (void)hipStreamSynchronize(stream);
      release(p);
      delete p;
      return st;
    }
    *out = p;
    return FFTMV_SUCCESS;
  } catch (...) {
    return FFTMV_ERR_INTERNAL;
  }
}

int fftmv_apply(fftmv_plan_t plan, const double *m_dev, double *v_dev, hipStream_t stream) {
  return apply_dir(plan, FFTMV_DIR_F, m_dev, v_dev, stream);
}

int fftmv_apply_adjoint(fftmv_plan_t plan, const double *d_dev, double *w_dev, hipStream_t stream) {
  return apply_dir(plan, FFTMV_DIR_FADJ, d_dev, w_dev, stream);
}

int fftmv_apply_scratch(fftmv_plan_t plan, int dir, const double *in, double *out, hipStream_t stream) {
  if ((dir != FFTMV_DIR_F && dir != FFTMV_DIR_FADJ) || !apply_args_ok(plan, dir, in, out))
    return FFTMV_ERR_INVALID_ARG;
  try {
    size_t need = 0;
    if (!scratch_layout(plan, dir, nullptr, nullptr, &need)) return FFTMV_ERR_UNSUPPORTED_SIZE;
    void *base = nullptr;
    hipError_t e = scratch_device_ptr(&base);
    if (e != hipSuccess) return status_from_hip(e);
    // the plan with its stage buffers and GEMV workspace in the scratch (a
    // copy of the plan's description; nothing is allocated or freed)
    fftmv_plan_s view = *plan;
    scratch_layout(plan, dir, static_cast<unsigned char *>(base), &view, &need);
    // The scratch keeps whatever the last call on this GPU left. The GEMV
    // reads the stage-2 spectrum in 16-byte vectors, which can cover the
    // padding entry after a row's last channel: those columns must hold
    // zeros (a kernel clears them; no memset node under stream capture).
    const StageBuf &b2 = view.buf[dir][2];
    const int64_t nin = channels_in(&view, dir);
    const int64_t esz2 = buf_f32(view.prec, dir, 2) ? 8 : 16;
    e = launch_zero_cols(b2.p, view.K, b2.ld * esz2, nin * esz2, (b2.ld - nin) * esz2, stream);
    if (e == hipSuccess) e = launch_apply(&view, dir, in, out, stream);
    return status_from_hip(e);
  } catch (...) {
    return FFTMV_ERR_INTERNAL;
  }
}

int fftmv_destroy(fftmv_plan_t plan) {
  if (!plan) return FFTMV_SUCCESS;
  int cur = 0;
  bool have_cur = hipGetDevice(&cur) == hipSuccess;
  (void)hipSetDevice(plan->device);
  hipError_t e = hipDeviceSynchronize();
  release(plan);
  if (have_cur) (void)hipSetDevice(cur);
  delete plan;
  return status_from_hip(e);
}

const char *fftmv_status_string(int status) {
  switch (status) {
    case FFTMV_SUCCESS: return "success";
    case FFTMV_ERR_INVALID_ARG: return "invalid argument";
    case FFTMV_ERR_UNSUPPORTED_SIZE:
      return "unsupported size (Nm above 2^27, Nd above 2^31 - 1, Nt above 4096, Nt above 2048 without a "
             "radix-2/3/5/7 factorisation, or a kernel grid above 2^32 work-items)";
    case FFTMV_ERR_OUT_OF_MEMORY: return "out of device memory";
    case FFTMV_ERR_HIP: return "HIP runtime error";
    case FFTMV_ERR_INTERNAL: return "internal error";
    case FFTMV_ERR_NO_CONFIG: return "no precision configuration meets the error tolerance";
    default: return "unknown status";
  }
}

int fftmv_query(fftmv_plan_t plan, size_t *fhat_bytes, size_t *workspace_bytes) {
  if (!plan) return FFTMV_ERR_INVALID_ARG;
  if (fhat_bytes) *fhat_bytes = plan->fhat_bytes;
  if (workspace_bytes) *workspace_bytes = plan->ws_bytes;
  return FFTMV_SUCCESS;
}

int fftmv_set_mask(fftmv_plan_t plan, uint32_t prec_mask) {
  if (!plan || (prec_mask & ~FFTMV_PREC_BITS) || !on_plan_device(plan)) return FFTMV_ERR_INVALID_ARG;
  if ((needs_fhat32(prec_mask) && !plan->fhat32) || (needs_fhat64(prec_mask) && !plan->fhat64))
    return FFTMV_ERR_INVALID_ARG;
  // Buffers change element type with the mask: clear them so that padding
  // entries read by the 16-byte vector loads hold zeros in the new layout.
  for (int dir = 0; dir < 2; ++dir)
    for (int st = 1; st <= 4; ++st) {
      const int64_t rows = (st == 1 || st == 4) ? plan->Nt : plan->K;
      const size_t bytes = static_cast<size_t>(rows * plan->buf[dir][st].ld) * ((st == 1 || st == 4) ? 8 : 16);
      if (hipMemset(plan->buf[dir][st].p, 0, bytes) != hipSuccess) return FFTMV_ERR_HIP;
    }
  if (hipDeviceSynchronize() != hipSuccess) return FFTMV_ERR_HIP;
  plan->prec = prec_mask;
  return FFTMV_SUCCESS;
}

int fftmv_run_stages(fftmv_plan_t plan, int dir, int first, int last, const double *in, double *out,
                     hipStream_t stream) {
  if (!plan || (dir != 0 && dir != 1) || first < 1 || last > 5 || first > last) return FFTMV_ERR_INVALID_ARG;
  if (first == 1 && (!in || !aligned8(in))) return FFTMV_ERR_INVALID_ARG;
  if (last == 5 && (!out || !aligned8(out))) return FFTMV_ERR_INVALID_ARG;
  if ((first == 1 && last == 5 && overlap(plan, dir, in, out)) || !on_plan_device(plan)) return FFTMV_ERR_INVALID_ARG;
  try {
    return status_from_hip(run_range(plan, dir, first, last, in, out, stream));
  } catch (...) {
    return FFTMV_ERR_INTERNAL;
  }
}

int fftmv_buffer(fftmv_plan_t plan, int which, void **ptr, int64_t *ld, int *elem_bytes) {
  if (!plan) return FFTMV_ERR_INVALID_ARG;
  void *q = nullptr;
  int64_t l = 0;
  int eb = 0;
  if (which == 0) {
    q = plan->fhat32, l = plan->ldF32, eb = 8;
  } else if (which == 1) {
    q = plan->fhat64, l = plan->ldF64, eb = 16;
  } else {
    const int dir = (which - 10) / 10, st = (which - 10) % 10;
    if (which < 10 || dir > 1 || st < 1 || st > 4) return FFTMV_ERR_INVALID_ARG;
    q = plan->buf[dir][st].p;
    l = plan->buf[dir][st].ld;
    const bool f32 = buf_f32(plan->prec, dir, st);
    eb = (st == 1 || st == 4) ? (f32 ? 4 : 8) : (f32 ? 8 : 16);
  }
  if (ptr) *ptr = q;
  if (ld) *ld = l;
  if (elem_bytes) *elem_bytes = eb;
  return FFTMV_SUCCESS;
}

int fftmv_condition(fftmv_plan_t plan, int iters, double *kappa, double *sigma_max, double *sigma_min,
                    hipStream_t stream) {
  if (!plan || !on_plan_device(plan)) return FFTMV_ERR_INVALID_ARG;
  try {
    return condition_impl(plan, iters, kappa, sigma_max, sigma_min, stream);
  } catch (...) {
    return FFTMV_ERR_INTERNAL;
  }
}

int fftmv_version(void) { return kVersion; }

}  // extern "C"
