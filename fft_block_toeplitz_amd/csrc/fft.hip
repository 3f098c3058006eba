// Batched real FFTs along time for the block-Toeplitz matvec: stage 2
// (forward, time -> frequency) and stage 4 (inverse, frequency -> time) of
// "Mixed-precision FFTMatvec performance optimization on AMD GPUs",
// section 1.1. The same forward kernel builds the frequency blocks at setup.
//
// A length N = 2L real transform is carried by one length-L complex
// transform of z[n] = x[2n] + i x[2n+1] (even samples in the real part, odd
// samples in the imaginary part), split afterwards with
//   X[k] = E[k] + w^k O[k],  E = (Z[k] + conj Z[L-k]) / 2,
//                            O = (Z[k] - conj Z[L-k]) / 2i,  w = exp(-2 pi i / N)
// and run backwards for the inverse. The zero half of the padded input
// (section 1.1, stage 1) is never loaded: samples at t >= Nt are zeros by
// construction; the inverse only produces the Nt samples the unpad keeps.
//
// One workgroup transforms C channels at once (C a power of two). The data
// sit in LDS as [L][C] complex, channel fastest, so consecutive lanes touch
// consecutive channels: global loads and stores along a time step or a
// frequency are contiguous over the C channels, and LDS accesses are
// stride-1 across lanes. The length-L complex FFT is a Stockham autosort
// (self-sorting, no bit reversal) with radix 2/4/5/8 passes; each pass reads
// all its butterfly inputs into registers, synchronises, then writes in
// place.
#include "common.hpp"
#include "internal.hpp"

namespace fftmv {
namespace {

// Butterflies a thread keeps in registers in one pass (bounded register
// use); the host picks C so that every pass fits.
template <typename T, int R>
constexpr int butterflies_per_thread() {
  if (sizeof(T) == 4) return R == 2 ? 16 : R == 4 ? 8 : R == 5 ? 7 : 4;
  return R == 2 ? 8 : R == 4 ? 4 : R == 5 ? 4 : 2;
}

int host_butterflies_per_thread(bool f32, int R) {
  if (f32) return R == 2 ? 16 : R == 4 ? 8 : R == 5 ? 7 : 4;
  return R == 2 ? 8 : R == 4 ? 4 : R == 5 ? 4 : 2;
}

// ---------------------------------------------------------------- DFTs
// y_q = sum_p x_p exp(S 2 pi i p q / R), in place, S = -1 forward, +1 inverse.
template <int S, typename T>
__device__ __forceinline__ void dft2(cx<T> &a, cx<T> &b) {
  cx<T> t = a - b;
  a = a + b;
  b = t;
}

template <int S, typename T>
__device__ __forceinline__ void dft4(cx<T> &x0, cx<T> &x1, cx<T> &x2, cx<T> &x3) {
  cx<T> t0 = x0 + x2, t1 = x0 - x2, t2 = x1 + x3, t3 = mul_si<S>(x1 - x3);
  x0 = t0 + t2;
  x2 = t0 - t2;
  x1 = t1 + t3;
  x3 = t1 - t3;
}

template <int S, typename T>
__device__ __forceinline__ void dft8(cx<T> *x) {
  // two length-4 transforms of the even and odd samples, then the
  // exp(S 2 pi i q / 8) twiddles and one radix-2 step
  const T h = T(0.70710678118654752440084436210484903928);  // 1/sqrt(2)
  dft4<S>(x[0], x[2], x[4], x[6]);
  dft4<S>(x[1], x[3], x[5], x[7]);
  cx<T> b1 = x[3], b2 = x[5], b3 = x[7];
  // positions: even transform a_q at x[0],x[2],x[4],x[6]; odd b_q at x[1],x[3],x[5],x[7]
  cx<T> a0 = x[0], a1 = x[2], a2 = x[4], a3 = x[6], b0 = x[1];
  b1 = mk((b1.re - S * b1.im) * h, (b1.im + S * b1.re) * h);   // * (1 + S i)/sqrt 2
  b2 = mul_si<S>(b2);                                          // * S i
  b3 = mk((-b3.re - S * b3.im) * h, (S * b3.re - b3.im) * h);  // * (-1 + S i)/sqrt 2
  x[0] = a0 + b0;
  x[4] = a0 - b0;
  x[1] = a1 + b1;
  x[5] = a1 - b1;
  x[2] = a2 + b2;
  x[6] = a2 - b2;
  x[3] = a3 + b3;
  x[7] = a3 - b3;
}

template <int S, typename T>
__device__ __forceinline__ void dft5(cx<T> *x) {
  // cos and sin of 2 pi / 5 and 4 pi / 5
  const T c1 = T(0.30901699437494742410229341718281905886);
  const T c2 = T(-0.80901699437494742410229341718281905886);
  const T s1 = T(0.95105651629515357211643933337938214340);
  const T s2 = T(0.58778525229247312916870595463907276860);
  cx<T> t1 = x[1] + x[4], t2 = x[2] + x[3], t3 = x[1] - x[4], t4 = x[2] - x[3];
  cx<T> a1 = mk(x[0].re + c1 * t1.re + c2 * t2.re, x[0].im + c1 * t1.im + c2 * t2.im);
  cx<T> a2 = mk(x[0].re + c2 * t1.re + c1 * t2.re, x[0].im + c2 * t1.im + c1 * t2.im);
  cx<T> b1 = mk(s1 * t3.re + s2 * t4.re, s1 * t3.im + s2 * t4.im);
  cx<T> b2 = mk(s2 * t3.re - s1 * t4.re, s2 * t3.im - s1 * t4.im);
  x[0] = x[0] + t1 + t2;
  b1 = mul_si<S>(b1);
  b2 = mul_si<S>(b2);
  x[1] = a1 + b1;
  x[4] = a1 - b1;
  x[2] = a2 + b2;
  x[3] = a2 - b2;
}

template <int R, int S, typename T>
__device__ __forceinline__ void dft(cx<T> *x) {
  if constexpr (R == 2) dft2<S>(x[0], x[1]);
  else if constexpr (R == 4) dft4<S>(x[0], x[1], x[2], x[3]);
  else if constexpr (R == 5) dft5<S>(x);
  else dft8<S>(x);
}

// One Stockham pass of radix R over the [L][C] LDS tile. Butterfly j of
// channel c reads elements j + q L/R, multiplies input q by
// w_{Ns R}^{(j mod Ns) q} and writes output q to (j - j mod Ns) R + j mod Ns + q Ns.
template <typename T, int R, int S>
__device__ __forceinline__ void stockham_pass(cx<T> *lds, int L, int logC, int Ns, int twstep,
                                              const cx<T> *__restrict__ tw) {
  constexpr int B = butterflies_per_thread<T, R>();
  const int C = 1 << logC;
  const int Lr = L / R;
  const int nb = Lr << logC;
  cx<T> v[B][R];
#pragma unroll
  for (int i = 0; i < B; ++i) {
    int b = threadIdx.x + i * kBlock;
    if (b < nb) {
      int c = b & (C - 1), j = b >> logC;
#pragma unroll
      for (int q = 0; q < R; ++q) v[i][q] = lds[((j + q * Lr) << logC) + c];
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < B; ++i) {
    int b = threadIdx.x + i * kBlock;
    if (b < nb) {
      int c = b & (C - 1), j = b >> logC;
      int k = j % Ns;
      if (Ns > 1) {
#pragma unroll
        for (int q = 1; q < R; ++q) {
          cx<T> w = tw[k * q * twstep];
          v[i][q] = S < 0 ? cmul(v[i][q], w) : cmulc(v[i][q], w);
        }
      }
      dft<R, S>(v[i]);
      int base = (j - k) * R + k;
#pragma unroll
      for (int q = 0; q < R; ++q) lds[((base + q * Ns) << logC) + c] = v[i][q];
    }
  }
  __syncthreads();
}

template <typename T, int S>
__device__ __forceinline__ void all_passes(cx<T> *lds, const FftGeom &g, int logC, const cx<T> *__restrict__ tw) {
  for (int p = 0; p < g.npass; ++p) {
    switch (g.radix[p]) {
      case 2: stockham_pass<T, 2, S>(lds, g.L, logC, g.ns[p], g.twstep[p], tw); break;
      case 4: stockham_pass<T, 4, S>(lds, g.L, logC, g.ns[p], g.twstep[p], tw); break;
      case 5: stockham_pass<T, 5, S>(lds, g.L, logC, g.ns[p], g.twstep[p], tw); break;
      default: stockham_pass<T, 8, S>(lds, g.L, logC, g.ns[p], g.twstep[p], tw); break;
    }
  }
}

template <typename T, typename Src, bool ROUND>
__device__ __forceinline__ T load_sample(const Src *p) {
  Src v = *p;
  if constexpr (ROUND && sizeof(Src) == 8) return static_cast<T>(round_f32(v));
  return static_cast<T>(v);
}

// --------------------------------------------------------------- forward
template <typename T, typename Src, bool ROUND>
__global__ __launch_bounds__(kBlock) void rfft_forward_kernel(FftGeom g, FwdFftArgs a, int logC,
                                                              const cx<T> *__restrict__ tw) {
  extern __shared__ __align__(16) unsigned char smem[];
  cx<T> *lds = reinterpret_cast<cx<T> *>(smem);
  const int C = 1 << logC;
  const int L = g.L;
  const int c = threadIdx.x & (C - 1);  // fixed per thread: kBlock is a multiple of C
  const int64_t ch = static_cast<int64_t>(blockIdx.x) * C + c;
  const bool live = ch < a.nchan;
  const Src *src = static_cast<const Src *>(a.src) + ch;

  // stages 1-2 boundary: packed samples z[n] = x[2n] + i x[2n+1]; samples at
  // t >= Nt are the zero padding and are not read
  for (int b = threadIdx.x; b < (L << logC); b += kBlock) {
    int64_t t0 = 2 * static_cast<int64_t>(b >> logC);
    T re = T(0), im = T(0);
    if (live && t0 < a.Nt) re = load_sample<T, Src, ROUND>(src + t0 * a.src_ld);
    if (live && t0 + 1 < a.Nt) im = load_sample<T, Src, ROUND>(src + (t0 + 1) * a.src_ld);
    lds[b] = mk(re, im);
  }
  __syncthreads();
  all_passes<T, -1>(lds, g, logC, tw);

  if (!live) return;
  const int64_t row = ch / a.cpr, col = ch - row * a.cpr;
  cx<float> *d32 = a.dst32 ? static_cast<cx<float> *>(a.dst32) + row * a.ldr32 + col : nullptr;
  cx<double> *d64 = a.dst64 ? static_cast<cx<double> *>(a.dst64) + row * a.ldr64 + col : nullptr;
  for (int b = threadIdx.x; b < ((L + 1) << logC); b += kBlock) {
    int k = b >> logC;
    int ka = k == L ? 0 : k, kb = k == 0 ? 0 : L - k;
    cx<T> za = lds[(ka << logC) + c], zb = conj(lds[(kb << logC) + c]);
    cx<T> e = scale(za + zb, T(0.5));
    cx<T> dd = za - zb;
    cx<T> o = mk(dd.im * T(0.5), -dd.re * T(0.5));  // (za - zb) / 2i
    cx<T> x = e + cmul(o, tw[k]);
    if (d64) d64[k * a.fstride64] = cvt<double>(x);
    if (d32) d32[k * a.fstride32] = cvt<float>(x);
  }
}

// --------------------------------------------------------------- inverse
template <typename T, typename Src>
__global__ __launch_bounds__(kBlock) void rfft_inverse_kernel(FftGeom g, InvFftArgs a, int logC,
                                                              const cx<T> *__restrict__ tw, T inv_l) {
  extern __shared__ __align__(16) unsigned char smem[];
  cx<T> *lds = reinterpret_cast<cx<T> *>(smem);
  const int C = 1 << logC;
  const int L = g.L;
  const int c = threadIdx.x & (C - 1);
  const int64_t ch = static_cast<int64_t>(blockIdx.x) * C + c;
  const bool live = ch < a.nchan;
  const cx<Src> *src = static_cast<const cx<Src> *>(a.src) + ch;

  // Z[k] = E[k] + i O[k] with E = (X[k] + conj X[L-k]) / 2 and
  // O = (X[k] - conj X[L-k]) conj(w^k) / 2; the imaginary parts of bins 0
  // and L (= Nt) are dropped, as a real signal's spectrum has none
  for (int b = threadIdx.x; b < (L << logC); b += kBlock) {
    int k = b >> logC;
    cx<T> z = mk(T(0), T(0));
    if (live) {
      cx<T> xa = cvt<T>(src[static_cast<int64_t>(k) * a.src_ld]);
      cx<T> xb = cvt<T>(src[static_cast<int64_t>(L - k) * a.src_ld]);
      if (k == 0) {
        xa.im = T(0);
        xb.im = T(0);
      }
      xb = conj(xb);
      cx<T> e = scale(xa + xb, T(0.5));
      cx<T> o = scale(cmulc(xa - xb, tw[k]), T(0.5));
      z = mk(e.re - o.im, e.im + o.re);
    }
    lds[b] = z;
  }
  __syncthreads();
  all_passes<T, +1>(lds, g, logC, tw);

  if (!live) return;
  // stage 4-5 boundary: z[n] = y[2n] + i y[2n+1]; keep t < Nt only
  const int64_t half = (a.Nt + 1) / 2;
  for (int b = threadIdx.x; b < (half << logC); b += kBlock) {
    int64_t n = b >> logC;
    cx<T> z = lds[b];
    T y0 = z.re * inv_l, y1 = z.im * inv_l;
    int64_t t0 = 2 * n;
    bool second = t0 + 1 < a.Nt;
    if (a.dst_f32) {
      float *d = static_cast<float *>(a.dst) + ch;
      d[t0 * a.dst_ld] = static_cast<float>(y0);
      if (second) d[(t0 + 1) * a.dst_ld] = static_cast<float>(y1);
    } else {
      double *d = static_cast<double *>(a.dst) + ch;
      double v0 = static_cast<double>(y0), v1 = static_cast<double>(y1);
      if (a.round_f32) {
        v0 = round_f32(v0);
        v1 = round_f32(v1);
      }
      d[t0 * a.dst_ld] = v0;
      if (second) d[(t0 + 1) * a.dst_ld] = v1;
    }
  }
}

int ilog2(int c) {
  int l = 0;
  while ((1 << l) < c) ++l;
  return l;
}

}  // namespace

int fft_channels_per_block(const FftGeom &g, bool f32, int64_t nchan) {
  const int64_t esz = f32 ? 8 : 16;
  int best = 0;
  for (int C = kMaxChannelsPerBlock; C >= 1; C >>= 1) {
    if (static_cast<int64_t>(g.L) * C * esz > kMaxLds) continue;
    bool ok = true;
    for (int p = 0; p < g.npass; ++p) {
      int64_t nb = static_cast<int64_t>(g.L / g.radix[p]) * C;
      if (nb > static_cast<int64_t>(host_butterflies_per_thread(f32, g.radix[p])) * kBlock) ok = false;
    }
    if (ok) {
      best = C;
      break;
    }
  }
  // Prefer more, narrower workgroups while the batch would not fill the GPU.
  while (best > 1 && (nchan + best - 1) / best < 512) best >>= 1;
  return best;
}

hipError_t launch_fft_forward(const FftGeom &g, const FwdFftArgs &a, bool compute_f32, const void *tw,
                              hipStream_t s) {
  const int C = fft_channels_per_block(g, compute_f32, a.nchan);
  if (C == 0) return hipErrorInvalidValue;
  const int logC = ilog2(C);
  const dim3 grid(static_cast<unsigned>((a.nchan + C - 1) / C));
  if (compute_f32) {
    const size_t lds = static_cast<size_t>(g.L) * C * sizeof(cx<float>);
    auto twp = static_cast<const cx<float> *>(tw);
    if (a.src_f32)
      hipLaunchKernelGGL((rfft_forward_kernel<float, float, false>), grid, dim3(kBlock), lds, s, g, a, logC, twp);
    else
      hipLaunchKernelGGL((rfft_forward_kernel<float, double, false>), grid, dim3(kBlock), lds, s, g, a, logC, twp);
  } else {
    const size_t lds = static_cast<size_t>(g.L) * C * sizeof(cx<double>);
    auto twp = static_cast<const cx<double> *>(tw);
    if (a.src_f32)
      hipLaunchKernelGGL((rfft_forward_kernel<double, float, false>), grid, dim3(kBlock), lds, s, g, a, logC, twp);
    else if (a.round_f32)
      hipLaunchKernelGGL((rfft_forward_kernel<double, double, true>), grid, dim3(kBlock), lds, s, g, a, logC, twp);
    else
      hipLaunchKernelGGL((rfft_forward_kernel<double, double, false>), grid, dim3(kBlock), lds, s, g, a, logC, twp);
  }
  return hipGetLastError();
}

hipError_t launch_fft_inverse(const FftGeom &g, const InvFftArgs &a, bool compute_f32, const void *tw,
                              hipStream_t s) {
  const int C = fft_channels_per_block(g, compute_f32, a.nchan);
  if (C == 0) return hipErrorInvalidValue;
  const int logC = ilog2(C);
  const dim3 grid(static_cast<unsigned>((a.nchan + C - 1) / C));
  if (compute_f32) {
    const size_t lds = static_cast<size_t>(g.L) * C * sizeof(cx<float>);
    auto twp = static_cast<const cx<float> *>(tw);
    const float inv_l = 1.0f / static_cast<float>(g.L);
    if (a.src_f32)
      hipLaunchKernelGGL((rfft_inverse_kernel<float, float>), grid, dim3(kBlock), lds, s, g, a, logC, twp, inv_l);
    else
      hipLaunchKernelGGL((rfft_inverse_kernel<float, double>), grid, dim3(kBlock), lds, s, g, a, logC, twp, inv_l);
  } else {
    const size_t lds = static_cast<size_t>(g.L) * C * sizeof(cx<double>);
    auto twp = static_cast<const cx<double> *>(tw);
    const double inv_l = 1.0 / static_cast<double>(g.L);
    if (a.src_f32)
      hipLaunchKernelGGL((rfft_inverse_kernel<double, float>), grid, dim3(kBlock), lds, s, g, a, logC, twp, inv_l);
    else
      hipLaunchKernelGGL((rfft_inverse_kernel<double, double>), grid, dim3(kBlock), lds, s, g, a, logC, twp, inv_l);
  }
  return hipGetLastError();
}

}  // namespace fftmv
