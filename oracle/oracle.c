/*
 * CPU oracle for the block-Toeplitz FFT matvec -- TEST INFRASTRUCTURE.
 *
 * Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load this library. The GPU library never links, includes or
 * calls it, and the two share no source, header, table or helper.
 *
 * Everything here is IEEE binary64 (the pages fix no precision for a
 * reference computation). It is deliberately plain: no blocking, no fusion,
 * sums run in index order.
 *
 * Source: "Mixed-precision FFTMatvec performance optimization on AMD GPUs"
 *   section 1    F is block triangular Toeplitz: block (i, j) is F_{i-j};
 *                read here as lower triangular (blocks with j > i are zero).
 *   section 1.1  the matvec runs in five stages: broadcast + zero pad, batched
 *                FFT (time -> frequency), block-diagonal matvec (SBGEMV),
 *                batched inverse FFT, unpad + reduce.
 *   section 1.2  the adjoint F* uses the conjugate transpose of each
 *                frequency block.
 *
 * Layouts (row-major):
 *   F    [Nt][Nd][Nm] double       block F_k at F + k*Nd*Nm
 *   m, w [Nt][Nm]     double       m_j is the j-th time step (block order)
 *   d, v [Nt][Nd]     double
 *   Fhat [Nt+1][Nd][Nm] complex    (re, im) pairs, frequency-major
 *   mhat [Nt+1][Nm] complex, vhat [Nt+1][Nd] complex (stage dumps)
 *
 * Readings of points the page leaves open:
 *   - zero padding appends Nt zeros (length N = 2 Nt) and the unpad keeps
 *     time steps 0..Nt-1; with the lower-triangular reading the circulant
 *     embedding then has no wrap-around;
 *   - forward DFT uses exp(-2 pi i n k / N) unnormalised, the inverse uses
 *     exp(+2 pi i n k / N) and a 1/N factor;
 *   - the half spectrum has K = Nt + 1 bins; the inverse rebuilds the other
 *     bins by Hermitian symmetry and keeps the real part, so the imaginary
 *     parts of bins 0 and Nt do not contribute;
 *   - broadcast and reduce over a processor grid are the identity on one
 *     processor.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    double re, im;
} cplx;

static inline cplx c_add(cplx a, cplx b) { cplx r = {a.re + b.re, a.im + b.im}; return r; }
static inline cplx c_mul(cplx a, cplx b) {
    cplx r = {a.re * b.re - a.im * b.im, a.re * b.im + a.im * b.re};
    return r;
}
static inline cplx c_conj(cplx a) { cplx r = {a.re, -a.im}; return r; }

enum { ORACLE_OK = 0, ORACLE_EINVAL = -1, ORACLE_ENOMEM = -2 };

/* ------------------------------------------------------------------------ */
/* Roots of unity                                                           */
/* ------------------------------------------------------------------------ */

/* tw[t] = exp(-2 pi i t / N), t = 0..N-1. The angle is formed from the exact
 * integer t < N and evaluated in long double, then rounded once to double. */
static cplx *roots_table(int64_t N) {
    static const long double two_pi = 6.283185307179586476925286766559005768L;
    cplx *tw = (cplx *)malloc((size_t)N * sizeof(cplx));
    if (!tw) return NULL;
    for (int64_t t = 0; t < N; ++t) {
        long double a = two_pi * (long double)t / (long double)N;
        tw[t].re = (double)cosl(a);
        tw[t].im = (double)(-sinl(a));
    }
    return tw;
}

/* exp(sign * 2 pi i * e / n) for an n dividing N, from the table for N. */
static inline cplx root(const cplx *tw, int64_t N, int64_t n, int64_t e, int sign) {
    cplx w = tw[(e % n) * (N / n)];
    return sign < 0 ? w : c_conj(w);
}

static int64_t smallest_prime_factor(int64_t n) {
    if (n % 2 == 0) return 2;
    for (int64_t p = 3; p * p <= n; p += 2)
        if (n % p == 0) return p;
    return n;
}

/* ------------------------------------------------------------------------ */
/* Recursive mixed-radix decimation-in-time FFT (Cooley and Tukey, 1965)     */
/* ------------------------------------------------------------------------ */

/* out[k] = sum_{j<n} in[j*stride] * exp(sign 2 pi i j k / n), k < n.
 * The smallest prime p of n is split off: the p decimated sequences
 * in[q + p j] (j < n/p) are transformed recursively into out[q*m .. q*m+m),
 * then X[k] = sum_q exp(sign 2 pi i q k / n) * Y_q[k mod m]. A prime n is
 * summed directly. scratch must hold n values. */
static void dft_rec(int64_t n, const cplx *in, int64_t stride, cplx *out, cplx *scratch,
                    const cplx *tw, int64_t N, int sign) {
    if (n == 1) {
        out[0] = in[0];
        return;
    }
    int64_t p = smallest_prime_factor(n);
    int64_t m = n / p;
    if (m == 1) {
        for (int64_t k = 0; k < n; ++k) {
            cplx s = {0.0, 0.0};
            for (int64_t j = 0; j < n; ++j)
                s = c_add(s, c_mul(in[j * stride], root(tw, N, n, j * k, sign)));
            scratch[k] = s;
        }
        memcpy(out, scratch, (size_t)n * sizeof(cplx));
        return;
    }
    for (int64_t q = 0; q < p; ++q)
        dft_rec(m, in + q * stride, stride * p, out + q * m, scratch, tw, N, sign);
    memcpy(scratch, out, (size_t)n * sizeof(cplx));
    for (int64_t k = 0; k < n; ++k) {
        cplx s = {0.0, 0.0};
        for (int64_t q = 0; q < p; ++q)
            s = c_add(s, c_mul(scratch[q * m + k % m], root(tw, N, n, q * k, sign)));
        out[k] = s;
    }
}

/* Unnormalised DFT of length n: sign = -1 forward, +1 inverse. */
int oracle_fft(int64_t n, const double *in, double *out, int sign) {
    if (n < 1 || !in || !out || (sign != 1 && sign != -1)) return ORACLE_EINVAL;
    cplx *tw = roots_table(n);
    cplx *scratch = (cplx *)malloc((size_t)n * sizeof(cplx));
    cplx *res = (cplx *)malloc((size_t)n * sizeof(cplx));
    if (!tw || !scratch || !res) {
        free(tw); free(scratch); free(res);
        return ORACLE_ENOMEM;
    }
    dft_rec(n, (const cplx *)in, 1, res, scratch, tw, n, sign);
    memcpy(out, res, (size_t)n * sizeof(cplx));
    free(tw); free(scratch); free(res);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Stage helpers                                                            */
/* ------------------------------------------------------------------------ */

/* Stages 1-2 for one channel: x = (s[0], .., s[Nt-1], 0, .., 0) of length
 * N = 2 Nt; X = DFT_N(x); returns X[0..Nt]. s is read with stride sstride. */
static void padded_forward(int64_t Nt, const double *s, int64_t sstride, cplx *Xhalf, cplx *xbuf,
                           cplx *ybuf, cplx *scratch, const cplx *tw) {
    int64_t N = 2 * Nt;
    for (int64_t n = 0; n < N; ++n) {
        xbuf[n].re = n < Nt ? s[n * sstride] : 0.0;
        xbuf[n].im = 0.0;
    }
    dft_rec(N, xbuf, 1, ybuf, scratch, tw, N, -1);
    memcpy(Xhalf, ybuf, (size_t)(Nt + 1) * sizeof(cplx));
}

/* Stages 4-5 for one channel: V[k] = Xhalf[k] for k <= Nt and
 * conj(Xhalf[N-k]) for k > Nt; y = Re(IDFT_N(V)) / N; returns y[0..Nt-1]
 * into t[i * tstride]. */
static void inverse_unpad(int64_t Nt, const cplx *Xhalf, double *t, int64_t tstride, cplx *xbuf,
                          cplx *ybuf, cplx *scratch, const cplx *tw) {
    int64_t N = 2 * Nt;
    for (int64_t k = 0; k < N; ++k)
        xbuf[k] = k <= Nt ? Xhalf[k] : c_conj(Xhalf[N - k]);
    dft_rec(N, xbuf, 1, ybuf, scratch, tw, N, +1);
    for (int64_t i = 0; i < Nt; ++i) t[i * tstride] = ybuf[i].re / (double)N;
}

static int dims_ok(int64_t Nm, int64_t Nd, int64_t Nt) { return Nm >= 1 && Nd >= 1 && Nt >= 1; }

/* ------------------------------------------------------------------------ */
/* Setup: the frequency blocks                                              */
/* ------------------------------------------------------------------------ */

/* Fhat[k][r][c] = sum_{n<Nt} F[n][r][c] exp(-2 pi i n k / (2 Nt)), k = 0..Nt:
 * the DFT of each zero-padded (r, c) series. */
int oracle_setup(const double *F, int64_t Nm, int64_t Nd, int64_t Nt, double *Fhat_out) {
    if (!F || !Fhat_out || !dims_ok(Nm, Nd, Nt)) return ORACLE_EINVAL;
    int64_t N = 2 * Nt, K = Nt + 1, C = Nd * Nm;
    cplx *tw = roots_table(N);
    if (!tw) return ORACLE_ENOMEM;
    cplx *Fhat = (cplx *)Fhat_out;
    int err = 0;
#pragma omp parallel
    {
        cplx *buf = (cplx *)malloc((size_t)(4 * N + K) * sizeof(cplx));
        if (!buf) {
#pragma omp atomic write
            err = 1;
        }
#pragma omp for schedule(static)
        for (int64_t ch = 0; ch < C; ++ch) {
            if (!buf) continue;
            cplx *xb = buf, *yb = buf + N, *sc = buf + 2 * N, *Xh = buf + 4 * N;
            padded_forward(Nt, F + ch, C, Xh, xb, yb, sc, tw);
            for (int64_t k = 0; k < K; ++k) Fhat[k * C + ch] = Xh[k];
        }
        free(buf);
    }
    free(tw);
    return err ? ORACLE_ENOMEM : ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* The five stages, forward: v = F m                                        */
/* ------------------------------------------------------------------------ */

/* Shared body of both directions. nin input channels, nout output channels;
 * adjoint selects the conjugate-transpose frequency product. */
static int five_stages(const cplx *Fhat, int64_t Nm, int64_t Nd, int64_t Nt, const double *in,
                       double *out, cplx *hin_dump, cplx *hout_dump, int adjoint) {
    int64_t N = 2 * Nt, K = Nt + 1;
    int64_t nin = adjoint ? Nd : Nm, nout = adjoint ? Nm : Nd;
    cplx *tw = roots_table(N);
    cplx *hin = (cplx *)malloc((size_t)(K * nin) * sizeof(cplx));
    cplx *hout = (cplx *)malloc((size_t)(K * nout) * sizeof(cplx));
    if (!tw || !hin || !hout) {
        free(tw); free(hin); free(hout);
        return ORACLE_ENOMEM;
    }
    int err = 0;

    /* Stages 1-2: pad each input channel with Nt zeros, forward DFT. */
#pragma omp parallel
    {
        cplx *buf = (cplx *)malloc((size_t)(4 * N + K) * sizeof(cplx));
        if (!buf) {
#pragma omp atomic write
            err = 1;
        }
#pragma omp for schedule(static)
        for (int64_t c = 0; c < nin; ++c) {
            if (!buf) continue;
            cplx *xb = buf, *yb = buf + N, *sc = buf + 2 * N, *Xh = buf + 4 * N;
            padded_forward(Nt, in + c, nin, Xh, xb, yb, sc, tw);
            for (int64_t k = 0; k < K; ++k) hin[k * nin + c] = Xh[k];
        }
        free(buf);
    }

    /* Stage 3: one complex matvec per frequency, sums in index order.
     * F:  vhat_k[r] = sum_c Fhat_k[r][c] mhat_k[c]
     * F*: what_k[c] = sum_r conj(Fhat_k[r][c]) dhat_k[r] */
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k) {
        const cplx *Fk = Fhat + k * Nd * Nm;
        const cplx *xk = hin + k * nin;
        cplx *yk = hout + k * nout;
        if (!adjoint) {
            for (int64_t r = 0; r < Nd; ++r) {
                cplx s = {0.0, 0.0};
                for (int64_t c = 0; c < Nm; ++c) s = c_add(s, c_mul(Fk[r * Nm + c], xk[c]));
                yk[r] = s;
            }
        } else {
            for (int64_t c = 0; c < Nm; ++c) yk[c].re = yk[c].im = 0.0;
            for (int64_t r = 0; r < Nd; ++r)
                for (int64_t c = 0; c < Nm; ++c)
                    yk[c] = c_add(yk[c], c_mul(c_conj(Fk[r * Nm + c]), xk[r]));
        }
    }

    /* Stages 4-5: inverse DFT of each output channel, keep time steps < Nt. */
#pragma omp parallel
    {
        cplx *buf = (cplx *)malloc((size_t)(4 * N + K) * sizeof(cplx));
        if (!buf) {
#pragma omp atomic write
            err = 1;
        }
#pragma omp for schedule(static)
        for (int64_t r = 0; r < nout; ++r) {
            if (!buf) continue;
            cplx *xb = buf, *yb = buf + N, *sc = buf + 2 * N, *Xh = buf + 4 * N;
            for (int64_t k = 0; k < K; ++k) Xh[k] = hout[k * nout + r];
            inverse_unpad(Nt, Xh, out + r, nout, xb, yb, sc, tw);
        }
        free(buf);
    }

    if (hin_dump) memcpy(hin_dump, hin, (size_t)(K * nin) * sizeof(cplx));
    if (hout_dump) memcpy(hout_dump, hout, (size_t)(K * nout) * sizeof(cplx));
    free(tw); free(hin); free(hout);
    return err ? ORACLE_ENOMEM : ORACLE_OK;
}

/* v = F m through the five stages. mhat_dump [K][Nm] and vhat_dump [K][Nd]
 * (complex) receive the stage-2 and stage-3 results when non-NULL. */
int oracle_apply(const double *Fhat, int64_t Nm, int64_t Nd, int64_t Nt, const double *m, double *v,
                 double *mhat_dump, double *vhat_dump) {
    if (!Fhat || !m || !v || !dims_ok(Nm, Nd, Nt)) return ORACLE_EINVAL;
    return five_stages((const cplx *)Fhat, Nm, Nd, Nt, m, v, (cplx *)mhat_dump, (cplx *)vhat_dump, 0);
}

/* w = F* d (the transpose, F being real) through the five stages with the
 * conjugate-transpose frequency product. */
int oracle_apply_adjoint(const double *Fhat, int64_t Nm, int64_t Nd, int64_t Nt, const double *d,
                         double *w, double *dhat_dump, double *what_dump) {
    if (!Fhat || !d || !w || !dims_ok(Nm, Nd, Nt)) return ORACLE_EINVAL;
    return five_stages((const cplx *)Fhat, Nm, Nd, Nt, d, w, (cplx *)dhat_dump, (cplx *)what_dump, 1);
}

/* ------------------------------------------------------------------------ */
/* The definition, summed directly                                          */
/* ------------------------------------------------------------------------ */

/* v_i[r] = sum_{j=0..i} sum_c F_{i-j}[r][c] m_j[c] for each listed step i.
 * v has [nsteps][Nd] entries, in the order of steps[]. */
int oracle_direct(const double *F, int64_t Nm, int64_t Nd, int64_t Nt, const double *m,
                  const int64_t *steps, int64_t nsteps, double *v) {
    if (!F || !m || !steps || !v || !dims_ok(Nm, Nd, Nt) || nsteps < 0) return ORACLE_EINVAL;
    for (int64_t s = 0; s < nsteps; ++s)
        if (steps[s] < 0 || steps[s] >= Nt) return ORACLE_EINVAL;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t s = 0; s < nsteps; ++s) {
        for (int64_t r = 0; r < Nd; ++r) {
            int64_t i = steps[s];
            double acc = 0.0;
            for (int64_t j = 0; j <= i; ++j) {
                const double *Frow = F + ((i - j) * Nd + r) * Nm;
                const double *mj = m + j * Nm;
                for (int64_t c = 0; c < Nm; ++c) acc += Frow[c] * mj[c];
            }
            v[s * Nd + r] = acc;
        }
    }
    return ORACLE_OK;
}

/* w_j[c] = sum_{i=j..Nt-1} sum_r F_{i-j}[r][c] d_i[r] for each listed step j.
 * w has [nsteps][Nm] entries. */
int oracle_direct_adjoint(const double *F, int64_t Nm, int64_t Nd, int64_t Nt, const double *d,
                          const int64_t *steps, int64_t nsteps, double *w) {
    if (!F || !d || !steps || !w || !dims_ok(Nm, Nd, Nt) || nsteps < 0) return ORACLE_EINVAL;
    for (int64_t s = 0; s < nsteps; ++s)
        if (steps[s] < 0 || steps[s] >= Nt) return ORACLE_EINVAL;
    /* Columns in blocks of 256 so that F is read along its rows; each
     * column's sum still runs over (i, r) in index order. */
    const int64_t CB = 256;
    int64_t ncb = (Nm + CB - 1) / CB;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t s = 0; s < nsteps; ++s) {
        for (int64_t cb = 0; cb < ncb; ++cb) {
            int64_t j = steps[s], c0 = cb * CB, c1 = c0 + CB < Nm ? c0 + CB : Nm;
            double acc[256];
            for (int64_t c = c0; c < c1; ++c) acc[c - c0] = 0.0;
            for (int64_t i = j; i < Nt; ++i)
                for (int64_t r = 0; r < Nd; ++r) {
                    const double *Frow = F + ((i - j) * Nd + r) * Nm;
                    double di = d[i * Nd + r];
                    for (int64_t c = c0; c < c1; ++c) acc[c - c0] += Frow[c] * di;
                }
            for (int64_t c = c0; c < c1; ++c) w[s * Nm + c] = acc[c - c0];
        }
    }
    return ORACLE_OK;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
