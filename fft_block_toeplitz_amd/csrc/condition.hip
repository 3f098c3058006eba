// Extreme singular values of the frequency blocks Fhat_k, for the condition
// number kappa(Fhat) that scales the error bound of "Mixed-precision
// FFTMatvec performance optimization on AMD GPUs", section 1.1 (the error
// predictor of section 2.1 starts from it).
//
// Fhat is block diagonal, so its singular values are those of all the
// Fhat_k together: kappa = max_k s_max(Fhat_k) / min_k s_min(Fhat_k), over
// the min(Nd, Nm) singular values of each block. Each block's extreme
// values come from a Lanczos process on its smaller Gram matrix G_k
// (Fhat_k Fhat_k^H when Nd <= Nm, else Fhat_k^H Fhat_k), all frequencies at
// once: the products with G_k are two launches of the library's own
// per-frequency GEMV kernels, and the kernels here do the rest -- one wave
// per frequency for the Lanczos recurrence (with full reorthogonalisation,
// classical Gram-Schmidt applied twice), then one thread per frequency for
// the extreme eigenvalues of the tridiagonal matrix by Sturm-count
// bisection.
#include "common.hpp"
#include "internal.hpp"

namespace fftmv {
namespace {

constexpr int kLanczosWave = 64;  // one wave per frequency

// splitmix64: a counter-based 64-bit mixer; gives the start vectors their
// generic (reproducible) components.
__device__ __forceinline__ uint64_t mix64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}
__device__ __forceinline__ double unit_uniform(uint64_t x) {  // [-1, 1)
  return static_cast<double>(mix64(x) >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}

__device__ __forceinline__ void put_x(void *x, int64_t idx, bool f32, cx<double> v) {
  if (f32)
    static_cast<cx<float> *>(x)[idx] = cvt<float>(v);
  else
    static_cast<cx<double> *>(x)[idx] = v;
}

// q_0 of every frequency: generic components, unit norm.
__global__ __launch_bounds__(kLanczosWave) void lanczos_start_kernel(LanczosArgs a) {
  const int64_t k = blockIdx.x;
  const int lane = threadIdx.x;
  cx<double> *q = reinterpret_cast<cx<double> *>(a.Q) + k * a.ldq;
  double ss = 0.0;
  for (int64_t i = lane; i < a.n; i += kLanczosWave) {
    const uint64_t c = 2 * static_cast<uint64_t>(k * a.n + i);
    const cx<double> v = mk(unit_uniform(c), unit_uniform(c + 1));
    q[i] = v;
    ss += v.re * v.re + v.im * v.im;
  }
  const double inv = 1.0 / sqrt(wave_sum(ss));
  for (int64_t i = lane; i < a.n; i += kLanczosWave) {
    const cx<double> v = scale(q[i], inv);
    q[i] = v;
    put_x(a.xin, k * a.ldx + i, a.x_f32, v);
  }
  if (lane == 0) a.len[k] = 0;
}

// <u, v> = sum conj(u_i) v_i over one frequency's vectors, uniform in the wave.
__device__ __forceinline__ cx<double> dotc(const cx<double> *u, const cx<double> *v, int64_t n, int lane) {
  double re = 0.0, im = 0.0;
  for (int64_t i = lane; i < n; i += kLanczosWave) {
    const cx<double> x = u[i], y = v[i];
    re += x.re * y.re + x.im * y.im;
    im += x.re * y.im - x.im * y.re;
  }
  return mk(wave_sum(re), wave_sum(im));
}

// Step j of the recurrence: z = G q_j on entry (overwritten),
//   alpha_j = <q_j, z>,  z -= alpha_j q_j + beta_{j-1} q_{j-1},
//   z -= sum_{i<=j} <q_i, z> q_i   (twice),
//   beta_j = |z|,  q_{j+1} = z / beta_j.
// A frequency stops when beta_j vanishes against the scale of its matrix
// (an invariant subspace: its Ritz values are then exact) or when its
// Krylov space is full (j + 1 == n); len[k] counts its completed steps.
__global__ __launch_bounds__(kLanczosWave) void lanczos_step_kernel(LanczosArgs a, int j) {
  const int64_t k = blockIdx.x;
  const int lane = threadIdx.x;
  if (a.len[k] != j) return;  // stopped at an earlier step
  __shared__ cx<double> h[kMaxLanczos];
  const int64_t qs = a.K * a.ldq;
  const cx<double> *Q = reinterpret_cast<const cx<double> *>(a.Q) + k * a.ldq;
  cx<double> *z = reinterpret_cast<cx<double> *>(a.z) + k * a.ldz;
  const cx<double> *qj = Q + j * qs;

  const double alpha = dotc(qj, z, a.n, lane).re;
  const double bprev = j > 0 ? a.beta[(j - 1) * a.K + k] : 0.0;
  for (int64_t i = lane; i < a.n; i += kLanczosWave) {
    cx<double> v = z[i] - scale(qj[i], alpha);
    if (j > 0) v = v - scale(Q[(j - 1) * qs + i], bprev);
    z[i] = v;
  }
  for (int pass = 0; pass < 2; ++pass) {
    for (int i = 0; i <= j; ++i) {
      const cx<double> c = dotc(Q + i * qs, z, a.n, lane);
      if (lane == 0) h[i] = c;
    }
    __syncthreads();
    for (int64_t e = lane; e < a.n; e += kLanczosWave) {
      cx<double> v = z[e];
      for (int i = 0; i <= j; ++i) v = v - cmul(h[i], Q[i * qs + e]);
      z[e] = v;
    }
    __syncthreads();
  }
  double ss = 0.0;
  for (int64_t i = lane; i < a.n; i += kLanczosWave) ss += z[i].re * z[i].re + z[i].im * z[i].im;
  const double beta = sqrt(wave_sum(ss));
  const bool stop = (j + 1 >= a.n) || !(beta > 1e-12 * (fabs(alpha) + bprev));
  if (!stop) {
    const double inv = 1.0 / beta;
    cx<double> *qn = reinterpret_cast<cx<double> *>(a.Q) + (j + 1) * qs + k * a.ldq;
    for (int64_t i = lane; i < a.n; i += kLanczosWave) {
      const cx<double> v = scale(z[i], inv);
      qn[i] = v;
      put_x(a.xin, k * a.ldx + i, a.x_f32, v);
    }
  }
  if (lane == 0) {
    a.alpha[j * a.K + k] = alpha;
    a.beta[j * a.K + k] = stop ? 0.0 : beta;
    a.len[k] = stop ? -(j + 1) : j + 1;  // negative: finished with j+1 steps
  }
}

// Number of eigenvalues below x of the symmetric tridiagonal matrix with
// diagonal alpha_0..alpha_{m-1} and off-diagonal beta_0..beta_{m-2} (Sturm
// sequence of the LDL^T pivots).
__device__ int sturm_count(const double *alpha, const double *beta, int64_t K, int m, double x, double pivmin) {
  int c = 0;
  double d = alpha[0] - x;
  if (fabs(d) < pivmin) d = -pivmin;
  c += d < 0.0;
  for (int i = 1; i < m; ++i) {
    const double b = beta[(i - 1) * K];
    d = (alpha[i * K] - x) - b * b / d;
    if (fabs(d) < pivmin) d = -pivmin;
    c += d < 0.0;
  }
  return c;
}

// Extreme eigenvalues of each frequency's Lanczos tridiagonal matrix;
// sigma[2k] = sqrt(lambda_max), sigma[2k+1] = sqrt(max(lambda_min, 0)).
__global__ void lanczos_extremes_kernel(LanczosArgs a, double *sigma) {
  const int64_t k = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (k >= a.K) return;
  const int m = a.len[k] < 0 ? -a.len[k] : a.len[k];
  const double *al = a.alpha + k, *be = a.beta + k;
  if (m == 0) {
    sigma[2 * k] = sigma[2 * k + 1] = 0.0;
    return;
  }
  double lo = al[0], hi = al[0], bmax = 0.0;
  for (int i = 0; i < m; ++i) {
    const double r = (i > 0 ? fabs(be[(i - 1) * a.K]) : 0.0) + (i + 1 < m ? fabs(be[i * a.K]) : 0.0);
    lo = fmin(lo, al[i * a.K] - r);
    hi = fmax(hi, al[i * a.K] + r);
    if (i + 1 < m) bmax = fmax(bmax, fabs(be[i * a.K]));
  }
  const double span = fmax(fabs(lo), fabs(hi));
  const double pivmin = fmax(span, bmax) * 1e-300 + 1e-300;
  lo -= 1e-14 * span + pivmin;
  hi += 1e-14 * span + pivmin;
  // lambda_min: the smallest x with one eigenvalue below it
  double l = lo, h = hi;
  for (int it = 0; it < 128 && h - l > 1e-16 * span; ++it) {
    const double mid = 0.5 * (l + h);
    if (sturm_count(al, be, a.K, m, mid, pivmin) >= 1) h = mid; else l = mid;
  }
  const double lmin = 0.5 * (l + h);
  l = lo, h = hi;
  for (int it = 0; it < 128 && h - l > 1e-16 * span; ++it) {
    const double mid = 0.5 * (l + h);
    if (sturm_count(al, be, a.K, m, mid, pivmin) >= m) h = mid; else l = mid;
  }
  const double lmax = 0.5 * (l + h);
  sigma[2 * k] = sqrt(fmax(lmax, 0.0));
  sigma[2 * k + 1] = sqrt(fmax(lmin, 0.0));
}

}  // namespace

hipError_t launch_lanczos_start(const LanczosArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(lanczos_start_kernel, dim3(static_cast<unsigned>(a.K)), dim3(kLanczosWave), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_lanczos_step(const LanczosArgs &a, int j, hipStream_t s) {
  if (j < 0 || j >= kMaxLanczos) return hipErrorInvalidValue;
  hipLaunchKernelGGL(lanczos_step_kernel, dim3(static_cast<unsigned>(a.K)), dim3(kLanczosWave), 0, s, a, j);
  return hipGetLastError();
}

hipError_t launch_lanczos_extremes(const LanczosArgs &a, double *sigma, hipStream_t s) {
  const unsigned blocks = static_cast<unsigned>((a.K + kBlock - 1) / kBlock);
  hipLaunchKernelGGL(lanczos_extremes_kernel, dim3(blocks), dim3(kBlock), 0, s, a, sigma);
  return hipGetLastError();
}

}  // namespace fftmv
