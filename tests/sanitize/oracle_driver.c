/* Runs the oracle (oracle/oracle.c) on small cases under AddressSanitizer and
 * UndefinedBehaviorSanitizer (CPU only). Every entry point is called, and
 * the results are cross-checked, so that a silent out-of-bounds access or
 * undefined operation that changes a result also fails here:
 *   - oracle_fft against the textbook DFT, both signs, n = 1..64 and 125;
 *   - the five-stage apply and adjoint against the direct sums at every
 *     time step, for shapes with odd, prime, power-of-two and unit sizes;
 *   - the adjoint identity <F m, d> = <m, F* d>.
 * Exit status 0 when every check passes. */
#define _USE_MATH_DEFINES
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_fft(int64_t n, const double *in, double *out, int sign);
int oracle_setup(const double *F, int64_t Nm, int64_t Nd, int64_t Nt, double *Fhat_out);
int oracle_apply(const double *Fhat, int64_t Nm, int64_t Nd, int64_t Nt, const double *m, double *v, double *mh,
                 double *vh);
int oracle_apply_adjoint(const double *Fhat, int64_t Nm, int64_t Nd, int64_t Nt, const double *d, double *w,
                         double *dh, double *wh);
int oracle_direct(const double *F, int64_t Nm, int64_t Nd, int64_t Nt, const double *m, const int64_t *steps,
                  int64_t nsteps, double *v);
int oracle_direct_adjoint(const double *F, int64_t Nm, int64_t Nd, int64_t Nt, const double *d,
                          const int64_t *steps, int64_t nsteps, double *w);
int oracle_num_threads(void);
void oracle_set_num_threads(int n);

#ifndef M_PI
#define M_PI 3.14159265358979323846
#endif

static uint64_t state = 0x9E3779B97F4A7C15ull;
static double uniform(void) { /* xorshift64*, in [-1, 1) */
  state ^= state >> 12;
  state ^= state << 25;
  state ^= state >> 27;
  return (double)((state * 0x2545F4914F6CDD1Dull) >> 11) / 4503599627370496.0 - 1.0;
}

static int failures = 0;
static void expect(int ok, const char *what, double value) {
  if (!ok) {
    fprintf(stderr, "FAILED: %s (%g)\n", what, value);
    ++failures;
  }
}

static double rel_diff(const double *a, const double *b, int64_t n) {
  double num = 0.0, den = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    num += (a[i] - b[i]) * (a[i] - b[i]);
    den += b[i] * b[i];
  }
  return den > 0.0 ? sqrt(num / den) : sqrt(num);
}

static void check_fft(int64_t n) {
  double *x = malloc(sizeof(double) * 2 * n), *y = malloc(sizeof(double) * 2 * n),
         *z = malloc(sizeof(double) * 2 * n);
  for (int64_t i = 0; i < 2 * n; ++i) x[i] = uniform();
  for (int sign = -1; sign <= 1; sign += 2) {
    expect(oracle_fft(n, x, y, sign) == 0, "oracle_fft status", (double)n);
    for (int64_t k = 0; k < n; ++k) { /* textbook DFT with the angle reduced in integers */
      double re = 0.0, im = 0.0;
      for (int64_t j = 0; j < n; ++j) {
        const double a = sign * 2.0 * M_PI * (double)((j * k) % n) / (double)n;
        re += x[2 * j] * cos(a) - x[2 * j + 1] * sin(a);
        im += x[2 * j] * sin(a) + x[2 * j + 1] * cos(a);
      }
      z[2 * k] = re;
      z[2 * k + 1] = im;
    }
    expect(rel_diff(y, z, 2 * n) <= 1e-12, "oracle_fft against the textbook DFT", rel_diff(y, z, 2 * n));
  }
  free(x);
  free(y);
  free(z);
}

static void check_apply(int64_t Nm, int64_t Nd, int64_t Nt) {
  const int64_t K = Nt + 1;
  double *F = malloc(sizeof(double) * Nt * Nd * Nm), *Fh = malloc(sizeof(double) * 2 * K * Nd * Nm);
  double *m = malloc(sizeof(double) * Nt * Nm), *d = malloc(sizeof(double) * Nt * Nd);
  double *v = malloc(sizeof(double) * Nt * Nd), *w = malloc(sizeof(double) * Nt * Nm);
  double *vd = malloc(sizeof(double) * Nt * Nd), *wd = malloc(sizeof(double) * Nt * Nm);
  double *mh = malloc(sizeof(double) * 2 * K * Nm), *vh = malloc(sizeof(double) * 2 * K * Nd);
  double *dh = malloc(sizeof(double) * 2 * K * Nd), *wh = malloc(sizeof(double) * 2 * K * Nm);
  int64_t *steps = malloc(sizeof(int64_t) * Nt);
  for (int64_t i = 0; i < Nt * Nd * Nm; ++i) F[i] = uniform();
  for (int64_t i = 0; i < Nt * Nm; ++i) m[i] = uniform();
  for (int64_t i = 0; i < Nt * Nd; ++i) d[i] = uniform();
  for (int64_t i = 0; i < Nt; ++i) steps[i] = i;
  expect(oracle_setup(F, Nm, Nd, Nt, Fh) == 0, "oracle_setup status", (double)Nt);
  expect(oracle_apply(Fh, Nm, Nd, Nt, m, v, mh, vh) == 0, "oracle_apply status", (double)Nt);
  expect(oracle_apply_adjoint(Fh, Nm, Nd, Nt, d, w, dh, wh) == 0, "oracle_apply_adjoint status", (double)Nt);
  expect(oracle_apply(Fh, Nm, Nd, Nt, m, v, NULL, NULL) == 0, "oracle_apply without dumps", (double)Nt);
  expect(oracle_direct(F, Nm, Nd, Nt, m, steps, Nt, vd) == 0, "oracle_direct status", (double)Nt);
  expect(oracle_direct_adjoint(F, Nm, Nd, Nt, d, steps, Nt, wd) == 0, "oracle_direct_adjoint status", (double)Nt);
  expect(rel_diff(v, vd, Nt * Nd) <= 1e-12, "apply against the direct sum", rel_diff(v, vd, Nt * Nd));
  expect(rel_diff(w, wd, Nt * Nm) <= 1e-12, "adjoint against the direct sum", rel_diff(w, wd, Nt * Nm));
  double a = 0.0, b = 0.0, na = 0.0, nb = 0.0;
  for (int64_t i = 0; i < Nt * Nd; ++i) a += v[i] * d[i], na += v[i] * v[i];
  for (int64_t i = 0; i < Nt * Nm; ++i) b += m[i] * w[i];
  for (int64_t i = 0; i < Nt * Nd; ++i) nb += d[i] * d[i];
  expect(fabs(a - b) <= 1e-12 * sqrt(na * nb), "adjoint identity", fabs(a - b));
  free(F), free(Fh), free(m), free(d), free(v), free(w), free(vd), free(wd);
  free(mh), free(vh), free(dh), free(wh), free(steps);
}

int main(void) {
  for (int64_t n = 1; n <= 64; ++n) check_fft(n);
  check_fft(125);
  const int64_t shapes[][3] = {{8, 4, 16}, {3, 5, 1}, {1, 1, 1}, {7, 3, 13}, {5, 2, 25}, {2, 6, 32}, {1, 3, 7}};
  const int threads = oracle_num_threads();
  for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i) check_apply(shapes[i][0], shapes[i][1], shapes[i][2]);
  oracle_set_num_threads(1); /* the same on one thread */
  check_apply(7, 3, 13);
  oracle_set_num_threads(threads);
  if (failures) return 1;
  printf("oracle under sanitizers: all checks passed\n");
  return 0;
}
