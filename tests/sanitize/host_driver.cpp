// Runs the host code of libfftmv (argument validation, plan construction
// up to its first device call, status strings, the precision model and
// selector) under AddressSanitizer and UndefinedBehaviorSanitizer, on a
// machine without a GPU: no call here reaches a kernel. The library is
// built with the sanitizers on its host code only (device code unchanged).
// Exit status 0 when every check passes.
#include <cmath>
#include <cstdint>
#include <cstdio>

#include "fftmv.h"

static int failures = 0;
static void expect(bool ok, const char *what, double value = 0.0) {
  if (!ok) {
    std::fprintf(stderr, "FAILED: %s (%g)\n", what, value);
    ++failures;
  }
}

int main() {
  // status strings and version
  for (int st = -10; st <= 1; ++st) expect(fftmv_status_string(st) != nullptr, "status string", st);
  expect(fftmv_version() > 0, "version");

  // setup: every invalid argument is rejected before device work
  void *const fake = reinterpret_cast<void *>(0x10000);
  const double *F = static_cast<const double *>(fake);
  struct Bad {
    const double *F;
    int64_t Nm, Nd, Nt;
    uint32_t mask;
    int status;
  } bad[] = {
      {nullptr, 8, 4, 16, 0, FFTMV_ERR_INVALID_ARG},
      {reinterpret_cast<const double *>(0x10004), 8, 4, 16, 0, FFTMV_ERR_INVALID_ARG},
      {F, 0, 4, 16, 0, FFTMV_ERR_INVALID_ARG},
      {F, 8, 0, 16, 0, FFTMV_ERR_INVALID_ARG},
      {F, 8, 4, 0, 0, FFTMV_ERR_INVALID_ARG},
      {F, -5, 4, 16, 0, FFTMV_ERR_INVALID_ARG},
      {F, 8, 4, 16, 1u << 12, FFTMV_ERR_INVALID_ARG},
      {F, 8, 4, 2053, 0, FFTMV_ERR_UNSUPPORTED_SIZE},
      {F, 8, 4, 4093, 0, FFTMV_ERR_UNSUPPORTED_SIZE},
      {F, 8, 4, 5000, 0, FFTMV_ERR_UNSUPPORTED_SIZE},
      {F, int64_t(1) << 31, 4, 16, 0, FFTMV_ERR_UNSUPPORTED_SIZE},
      {F, (int64_t(1) << 27) + 1, 4, 16, 0, FFTMV_ERR_UNSUPPORTED_SIZE},
      {F, 8, int64_t(1) << 40, 16, 0, FFTMV_ERR_UNSUPPORTED_SIZE},
  };
  for (const Bad &b : bad) {
    fftmv_plan_t plan = nullptr;
    expect(fftmv_setup(&plan, b.F, b.Nm, b.Nd, b.Nt, b.mask, nullptr) == b.status, "setup validation", b.Nt);
    expect(plan == nullptr, "no plan on failure");
  }
  expect(fftmv_setup(nullptr, F, 8, 4, 16, 0, nullptr) == FFTMV_ERR_INVALID_ARG, "setup without out");
  // valid arguments reach plan construction (radix, Bluestein and fixed
  // lengths) and fail at the first device call on a machine without a GPU,
  // releasing what they built
  const int64_t lengths[] = {1, 7, 13, 16, 1000, 1009, 2000, 3920, 4096};
  for (int64_t Nt : lengths) {
    fftmv_plan_t plan = nullptr;
    const int st = fftmv_setup(&plan, F, 37, 5, Nt, FFTMV_MIXED | FFTMV_FLAG_FHAT_BOTH, nullptr);
    expect(st != FFTMV_SUCCESS && plan == nullptr, "setup without a device fails cleanly", Nt);
  }

  // every plan entry point rejects a null plan
  const double *in = static_cast<const double *>(fake);
  double *out = static_cast<double *>(fake);
  expect(fftmv_apply(nullptr, in, out, nullptr) == FFTMV_ERR_INVALID_ARG, "apply null plan");
  expect(fftmv_apply_adjoint(nullptr, in, out, nullptr) == FFTMV_ERR_INVALID_ARG, "adjoint null plan");
  expect(fftmv_apply_scratch(nullptr, 0, in, out, nullptr) == FFTMV_ERR_INVALID_ARG, "scratch null plan");
  expect(fftmv_query(nullptr, nullptr, nullptr) == FFTMV_ERR_INVALID_ARG, "query null plan");
  expect(fftmv_set_mask(nullptr, 0) == FFTMV_ERR_INVALID_ARG, "set_mask null plan");
  expect(fftmv_run_stages(nullptr, 0, 1, 5, in, out, nullptr) == FFTMV_ERR_INVALID_ARG, "run_stages null plan");
  expect(fftmv_buffer(nullptr, 0, nullptr, nullptr, nullptr) == FFTMV_ERR_INVALID_ARG, "buffer null plan");
  expect(fftmv_condition(nullptr, 0, nullptr, nullptr, nullptr, nullptr) == FFTMV_ERR_INVALID_ARG,
         "condition null plan");
  expect(fftmv_destroy(nullptr) == FFTMV_SUCCESS, "destroy null plan");

  // precision model: defaults, predictions over shapes and configurations,
  // the Pareto front and the selection, and parameter validation
  double params[2][FFTMV_MODEL_PARAMS];
  for (int dir = 0; dir < 2; ++dir) expect(fftmv_model_defaults(dir, params[dir]) == FFTMV_SUCCESS, "defaults");
  expect(fftmv_model_defaults(2, params[0]) == FFTMV_ERR_INVALID_ARG, "defaults bad direction");
  expect(fftmv_model_defaults(0, nullptr) == FFTMV_ERR_INVALID_ARG, "defaults null");
  const int64_t shapes[][3] = {{5000, 100, 1000}, {1, 1, 1}, {20000, 100, 2000}, {8, 4, 16},
                               {4, 100000, 1000}, {700, 3, 1029}, {37, 5, 1009}, {3, 2, 4096}};
  const double kappas[] = {1.0, 1.3, 1e4, 1e12};
  const double tols[] = {1e-15, 1e-11, 1e-7, 1e-6, 1e-3, 1.0};
  for (const auto &sh : shapes)
    for (int dir = 0; dir < 2; ++dir)
      for (uint32_t flags : {0u, static_cast<uint32_t>(FFTMV_FLAG_STAGED)})
        for (double kappa : kappas) {
          for (uint32_t bits = 0; bits < 32; ++bits) {
            double e = -1.0, t = -1.0;
            expect(fftmv_predict(sh[0], sh[1], sh[2], dir, bits, flags, kappa, nullptr, &e, &t) == FFTMV_SUCCESS,
                   "predict", bits);
            expect(std::isfinite(e) && e > 0.0 && std::isfinite(t) && t > 0.0, "finite prediction", e);
          }
          for (double tol : tols) {
            uint32_t front[32];
            int count = -1;
            expect(fftmv_pareto_front(sh[0], sh[1], sh[2], dir, flags, kappa, tol, params[dir], front, &count) ==
                       FFTMV_SUCCESS,
                   "pareto front", tol);
            expect(count >= 0 && count <= 32, "front size", count);
            for (int i = 0; i < count; ++i) expect(front[i] < 32u, "front entry", front[i]);
            uint32_t pick = 99;
            double e = 0.0, t = 0.0;
            const int st = fftmv_select_precision(sh[0], sh[1], sh[2], dir, flags, kappa, tol, nullptr, &pick, &e, &t);
            expect(st == FFTMV_SUCCESS || st == FFTMV_ERR_NO_CONFIG, "select status", st);
            expect(pick < 32u && (st == FFTMV_SUCCESS || pick == 0u), "selected configuration", pick);
          }
        }
  double e = 0.0, t = 0.0;
  expect(fftmv_predict(5000, 100, 1000, 0, 32, 0, 1.0, nullptr, &e, &t) == FFTMV_ERR_INVALID_ARG, "bits > 31");
  expect(fftmv_predict(5000, 100, 1000, 0, 6, 0, std::nan(""), nullptr, &e, &t) == FFTMV_ERR_INVALID_ARG, "NaN kappa");
  expect(fftmv_predict(5000, 100, 1000, 0, 6, 0, 0.5, nullptr, &e, &t) == FFTMV_ERR_INVALID_ARG, "kappa < 1");
  expect(fftmv_predict(5000, 100, 1000, 0, 6, 1u << 20, 1.0, nullptr, &e, &t) == FFTMV_ERR_INVALID_ARG, "bad flag");
  expect(fftmv_predict(5000, 100, 4093, 0, 6, 0, 1.0, nullptr, &e, &t) == FFTMV_ERR_UNSUPPORTED_SIZE, "bad length");
  double badp[FFTMV_MODEL_PARAMS];
  for (int i = 0; i < FFTMV_MODEL_PARAMS; ++i) badp[i] = params[0][i];
  badp[6] = 0.0;  // zero bandwidth
  expect(fftmv_predict(5000, 100, 1000, 0, 6, 0, 1.0, badp, &e, &t) == FFTMV_ERR_INVALID_ARG, "zero bandwidth");
  badp[6] = params[0][6];
  badp[0] = -1.0;  // negative constant
  expect(fftmv_predict(5000, 100, 1000, 0, 6, 0, 1.0, badp, &e, &t) == FFTMV_ERR_INVALID_ARG, "negative constant");
  uint32_t front[32];
  int count = 0;
  expect(fftmv_pareto_front(5000, 100, 1000, 0, 0, 1.0, 1e-6, nullptr, nullptr, &count) == FFTMV_ERR_INVALID_ARG,
         "front null");
  expect(fftmv_pareto_front(5000, 100, 1000, 0, 0, 1.0, std::nan(""), nullptr, front, &count) ==
             FFTMV_ERR_INVALID_ARG,
         "front NaN tolerance");

  if (failures) return 1;
  std::printf("library host code under sanitizers: all checks passed\n");
  return 0;
}
