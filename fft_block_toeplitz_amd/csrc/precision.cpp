// Precision selection of "Mixed-precision FFTMatvec performance optimization
// on AMD GPUs": the error bound of section 1.1 as the error predictor, a
// bandwidth model as the performance predictor, and the Pareto search of
// section 2.1 over the 32 stage configurations of section 2.2. Host only.
#include <algorithm>
#include <cmath>
#include <cstdint>

#include "fftmv.h"
#include "internal.hpp"

using fftmv::make_geometry;

namespace {

constexpr double kU32 = 5.9604644775390625e-08;  // 2^-24, binary32 unit roundoff
constexpr double kU64 = 1.1102230246251565e-16;  // 2^-53, binary64 unit roundoff

// c1..c5, cF, B (bytes/s), B_lds (bytes/s), t0 (s) per direction. The
// constants come from the 32-configuration sweep of each direction on one
// MI355X at Nm=5000, Nd=100, Nt=1000 (each c_s from the configuration with
// stage s alone in FP32, then all scaled so that the bound holds for every
// configuration of the sweep); B, B_lds and t0 are a least-squares fit of
// the measured apply times. F*'s time parameters come from an earlier sweep
// of the same kernels' bytes: a refit after the conjugate-transpose GEMV
// gained its row sub-sums dropped the LDS term (no cost for an FP64 inverse
// FFT), which ranks the SBGEMV alone in FP32 ahead of FFT + SBGEMV + IFFT
// in FP32 at a 1e-6 tolerance although the latter measures 1.7% faster.
constexpr double kDefaults[2][FFTMV_MODEL_PARAMS] = {
    {0.3167, 0.1233, 0.0002352, 0.1566, 0.3162, 1, 6.9006e+12, 3.0736e+13, 0.0000e+00},  // F
    {0.3176, 0.1239, 0.01035, 0.1557, 0.3156, 1, 6.5961e+12, 6.1142e+13, 0.0000e+00},  // F*
};

struct Problem {
  double Nm, Nd, Nt;
  int dir;
};

bool fp32(uint32_t bits, int stage) { return (bits >> (stage - 1)) & 1u; }
double unit_roundoff(uint32_t bits, int stage) { return fp32(bits, stage) ? kU32 : kU64; }

// The bound of section 1.1 with pc = 1 (one GPU); the stage-5 term keeps the
// one rounding of the output (max(1, log2 pc) = 1).
double predict_error(const Problem &p, uint32_t bits, double kappa, const double *c) {
  const double lg = std::log2(p.Nt);
  const double n = p.dir == 0 ? p.Nm : p.Nd;
  const double fft = c[5] * kU64 + c[1] * unit_roundoff(bits, 2) + c[3] * unit_roundoff(bits, 4);
  return kappa * (c[0] * unit_roundoff(bits, 1) + fft * lg + c[2] * unit_roundoff(bits, 3) * n +
                  c[4] * unit_roundoff(bits, 5));
}

bool radix_fits(int64_t Nt);

// HBM: algorithmic bytes of each kernel of one apply; a buffer between
// stages s and s+1 holds the narrower of their precisions. LDS: each pass of
// a batched FFT writes and reads its tile of Nt complex values per channel
// (in Bluestein form: two transforms of M values) in the precision of its
// stage.
double predict_seconds(const Problem &p, uint32_t bits, bool staged, const double *c) {
  const double K = p.Nt + 1.0;
  const double nin = p.dir == 0 ? p.Nm : p.Nd, nout = p.dir == 0 ? p.Nd : p.Nm;
  auto real_bytes = [&](int s) { return fp32(bits, s) || fp32(bits, s + 1) ? 4.0 : 8.0; };
  const double fhat = K * p.Nd * p.Nm * (fp32(bits, 3) ? 8.0 : 16.0);
  const double hin = K * nin * 2.0 * real_bytes(2);    // forward spectrum
  const double hout = K * nout * 2.0 * real_bytes(3);  // product spectrum
  double bytes = 0.0;
  int kernels = 0;
  if (staged) {
    const double x = p.Nt * nin * real_bytes(1), y = p.Nt * nout * real_bytes(4);
    bytes = (p.Nt * nin * 8.0 + x) + (x + hin) + (fhat + hin + hout) + (hout + y) + (y + p.Nt * nout * 8.0);
    kernels = 5;
  } else {
    bytes = (p.Nt * nin * 8.0 + hin) + (fhat + hin + hout) + (hout + p.Nt * nout * 8.0);
    kernels = 3;
  }
  const int64_t Nt = static_cast<int64_t>(p.Nt);
  double tile_passes = 0.0;  // passes times tile length, per channel
  if (radix_fits(Nt)) {
    tile_passes = make_geometry(static_cast<int>(Nt)).npass * p.Nt;
  } else {
    const int64_t M = fftmv::bluestein_length(Nt);
    tile_passes = 2.0 * make_geometry(static_cast<int>(M)).npass * static_cast<double>(M);
  }
  const double lds = 2.0 * tile_passes * (nin * (fp32(bits, 2) ? 8.0 : 16.0) + nout * (fp32(bits, 4) ? 8.0 : 16.0));
  return bytes / c[6] + lds / c[7] + kernels * c[8];
}

// the sizes fftmv_setup accepts: a radix schedule that fits a workgroup,
// else the Bluestein form
bool radix_fits(int64_t Nt) {
  const fftmv::FftGeom g = make_geometry(static_cast<int>(Nt));
  return g.L == Nt && fftmv::fft_channels_per_block(g, false, 1) > 0 && fftmv::fft_channels_per_block(g, true, 1) > 0;
}
bool supported(int64_t Nt) {
  if (Nt < 1 || Nt > 4096) return false;
  return radix_fits(Nt) || fftmv::bluestein_length(Nt) > 0;
}

bool valid(int64_t Nm, int64_t Nd, int64_t Nt, int dir, uint32_t flags, double kappa, const double *c) {
  if (Nm < 1 || Nd < 1 || Nt < 1 || (dir != 0 && dir != 1)) return false;
  if (flags & ~static_cast<uint32_t>(FFTMV_FLAG_BITS)) return false;
  if (!(kappa >= 1.0)) return false;  // also rejects NaN
  if (c) {
    for (int i = 0; i < 6; ++i)
      if (!(c[i] >= 0.0) || !std::isfinite(c[i])) return false;
    for (int i = 6; i < 8; ++i)
      if (!(c[i] > 0.0)) return false;  // bandwidths: positive, may be +Inf
    if (!(c[8] >= 0.0) || !std::isfinite(c[8])) return false;
  }
  return true;
}

struct Candidate {
  uint32_t bits;
  double err, sec;
};

int popcount5(uint32_t b) { return __builtin_popcount(b & 31u); }

// faster first; then more accurate; then fewer FP32 stages; then by value
bool before(const Candidate &a, const Candidate &b) {
  if (a.sec != b.sec) return a.sec < b.sec;
  if (a.err != b.err) return a.err < b.err;
  if (popcount5(a.bits) != popcount5(b.bits)) return popcount5(a.bits) < popcount5(b.bits);
  return a.bits < b.bits;
}

// Feasible Pareto front, in the order of `before`. Returns its length.
int pareto(const Problem &p, uint32_t flags, double kappa, double tol, const double *c, Candidate *front) {
  Candidate all[32];
  int n = 0;
  for (uint32_t b = 0; b < 32; ++b) {
    const Candidate x{b, predict_error(p, b, kappa, c), predict_seconds(p, b, flags & FFTMV_FLAG_STAGED, c)};
    if (x.err <= tol) all[n++] = x;
  }
  std::sort(all, all + n, before);
  // walking in time order, a candidate is on the front when it is strictly
  // more accurate than everything before it (equal time and error: the
  // first in order represents them)
  int m = 0;
  double best_err = INFINITY;
  for (int i = 0; i < n; ++i) {
    if (all[i].err < best_err) {
      front[m++] = all[i];
      best_err = all[i].err;
    }
  }
  return m;
}

}  // namespace

extern "C" {

int fftmv_model_defaults(int dir, double *params) {
  if ((dir != 0 && dir != 1) || !params) return FFTMV_ERR_INVALID_ARG;
  std::copy(kDefaults[dir], kDefaults[dir] + FFTMV_MODEL_PARAMS, params);
  return FFTMV_SUCCESS;
}

int fftmv_predict(int64_t Nm, int64_t Nd, int64_t Nt, int dir, uint32_t stage_bits, uint32_t flags, double kappa,
                  const double *params, double *est_error, double *est_seconds) {
  if (!valid(Nm, Nd, Nt, dir, flags, kappa, params) || stage_bits > 31u) return FFTMV_ERR_INVALID_ARG;
  if (!supported(Nt)) return FFTMV_ERR_UNSUPPORTED_SIZE;
  const double *c = params ? params : kDefaults[dir];
  const Problem p{static_cast<double>(Nm), static_cast<double>(Nd), static_cast<double>(Nt), dir};
  if (est_error) *est_error = predict_error(p, stage_bits, kappa, c);
  if (est_seconds) *est_seconds = predict_seconds(p, stage_bits, flags & FFTMV_FLAG_STAGED, c);
  return FFTMV_SUCCESS;
}

int fftmv_pareto_front(int64_t Nm, int64_t Nd, int64_t Nt, int dir, uint32_t flags, double kappa, double error_tol,
                       const double *params, uint32_t *front, int *count) {
  if (!valid(Nm, Nd, Nt, dir, flags, kappa, params) || !front || !count || std::isnan(error_tol))
    return FFTMV_ERR_INVALID_ARG;
  if (!supported(Nt)) return FFTMV_ERR_UNSUPPORTED_SIZE;
  const double *c = params ? params : kDefaults[dir];
  const Problem p{static_cast<double>(Nm), static_cast<double>(Nd), static_cast<double>(Nt), dir};
  Candidate f[32];
  const int m = pareto(p, flags, kappa, error_tol, c, f);
  for (int i = 0; i < m; ++i) front[i] = f[i].bits;
  *count = m;
  return FFTMV_SUCCESS;
}

int fftmv_select_precision(int64_t Nm, int64_t Nd, int64_t Nt, int dir, uint32_t flags, double kappa,
                           double error_tol, const double *params, uint32_t *stage_bits, double *est_error,
                           double *est_seconds) {
  if (!valid(Nm, Nd, Nt, dir, flags, kappa, params) || std::isnan(error_tol)) return FFTMV_ERR_INVALID_ARG;
  if (!supported(Nt)) return FFTMV_ERR_UNSUPPORTED_SIZE;
  const double *c = params ? params : kDefaults[dir];
  const Problem p{static_cast<double>(Nm), static_cast<double>(Nd), static_cast<double>(Nt), dir};
  Candidate f[32];
  const int m = pareto(p, flags, kappa, error_tol, c, f);
  const Candidate pick =
      m > 0 ? f[0] : Candidate{0u, predict_error(p, 0u, kappa, c), predict_seconds(p, 0u, flags & FFTMV_FLAG_STAGED, c)};
  if (stage_bits) *stage_bits = pick.bits;
  if (est_error) *est_error = pick.err;
  if (est_seconds) *est_seconds = pick.sec;
  return m > 0 ? FFTMV_SUCCESS : FFTMV_ERR_NO_CONFIG;
}

}  // extern "C"
