/*
 * fftmv -- block lower-triangular Toeplitz matvec through the FFT, on one
 * AMD Instinct MI355X (gfx950).
 *
 * Operation ("Mixed-precision FFTMatvec performance optimization on AMD
 * GPUs", sections 1 and 1.1): F is an Nt x Nt grid of blocks, block (i, j)
 * being the Nd x Nm matrix F_{i-j} for i >= j and zero above the diagonal.
 *
 *     v = F m      v_i = sum_{j <= i}     F_{i-j}   m_j     (i < Nt)
 *     w = F* d     w_j = sum_{i >= j}     F_{i-j}^T d_i     (j < Nt)
 *
 * Both run in the page's five stages: (1) broadcast + zero pad each channel
 * to length N = 2 Nt, (2) batched real FFT, (3) one complex GEMV per
 * frequency k = 0..Nt against the precomputed frequency blocks
 * Fhat_k = sum_n F_n exp(-2 pi i n k / N) -- the conjugate transpose
 * Fhat_k^H for F* (section 1.2) -- (4) batched inverse real FFT, (5) unpad
 * (keep time steps 0..Nt-1) and reduce. On one GPU the broadcast and the
 * reduce are the identity.
 *
 * Mixed precision (section 2.2): each of the five stages of each direction
 * runs in FP32 or FP64, chosen by a 10-bit mask. The page's configurations
 * for a 1e-7 error budget are FFTMV_MIXED_F (FFT + SBGEMV in FP32) and
 * FFTMV_MIXED_FADJ (SBGEMV + inverse FFT in FP32).
 *
 * Layouts (row-major, all device memory, FP64 at the interface):
 *   F    [Nt][Nd][Nm]   block F_k starts at F + k*Nd*Nm
 *   m, w [Nt][Nm]       time step j is the contiguous Nm-vector m + j*Nm
 *   d, v [Nt][Nd]
 * Pointers need 8-byte alignment (natural for double).
 *
 * Supported sizes: 1 <= Nm <= 2^27 (a complex128 row of Fhat within 2 GiB),
 * 1 <= Nd <= 2^31 - 1, and 1 <= Nt <= 4096 where
 *   - Nt = 2^a 3^b 5^c 7^d runs with radix 2/4/8, 3, 5 and 7 passes, and
 *   - any other Nt <= 2048 runs in Bluestein (chirp-z) form: the length-Nt
 *     transform as a circular convolution of a power-of-two length
 *     M >= 2 Nt - 1;
 * any other size returns FFTMV_ERR_UNSUPPORTED_SIZE. So does a launch whose
 * grid would exceed the 2^32 work-items of one dispatch, which only the
 * largest batches near the memory limit reach (e.g. the setup transform of
 * more than ~4 million channels at Nt = 4096); setup reports it for the
 * transforms, an apply for its GEMV kernels.
 *
 * Ownership and concurrency:
 *   - fftmv_setup is synchronous: when it returns the frequency blocks are
 *     built and the caller may free F. The plan owns Fhat, its twiddle
 *     tables and one workspace, all in device memory.
 *   - fftmv_apply / fftmv_apply_adjoint are asynchronous on the stream they
 *     are given; they allocate nothing and never synchronise. The caller owns
 *     the vectors and the streams. An output that overlaps its input is
 *     rejected with FFTMV_ERR_INVALID_ARG.
 *   - A plan lives on the device current at fftmv_setup. Every call that
 *     launches work with it (applies, fftmv_run_stages, fftmv_set_mask,
 *     fftmv_condition) needs that device current, else it returns
 *     FFTMV_ERR_INVALID_ARG without launching anything.
 *   - Applies on one plan share its workspace: they must be ordered (one
 *     stream, or caller synchronisation). Different plans are independent.
 *
 * Errors: every entry point returns FFTMV_SUCCESS (0) or a negative status.
 * Arguments are checked before any device work; no C++ exception crosses
 * this interface. A fault inside a kernel surfaces at the caller's next
 * synchronisation of the stream, as usual in HIP. NaN and Inf inputs are
 * not masked: they propagate (the FFT spreads them over their channel).
 */
#ifndef FFTMV_H
#define FFTMV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef FFTMV_API
#define FFTMV_API __attribute__((visibility("default")))
#endif

/* ----------------------------------------------------------------- status */
#define FFTMV_SUCCESS 0
#define FFTMV_ERR_INVALID_ARG (-1)      /* null pointer, bad size/mask/stage  */
#define FFTMV_ERR_UNSUPPORTED_SIZE (-2) /* size outside the supported range   */
#define FFTMV_ERR_OUT_OF_MEMORY (-3)    /* device allocation failed           */
#define FFTMV_ERR_HIP (-4)              /* a HIP runtime call or launch failed */
#define FFTMV_ERR_INTERNAL (-5)         /* unexpected library condition       */
#define FFTMV_ERR_NO_CONFIG (-6)        /* no precision configuration meets the
                                           error tolerance                    */

/* ------------------------------------------------------- precision mask
 * Bit (5*dir + stage - 1) set = that stage runs in FP32, clear = FP64.
 * dir 0 is F, dir 1 is F*; stages are numbered in pipeline order:
 * 1 pad, 2 forward FFT, 3 SBGEMV, 4 inverse FFT, 5 unpad. */
#define FFTMV_DIR_F 0
#define FFTMV_DIR_FADJ 1
#define FFTMV_FP32(dir, stage) (1u << (5u * (unsigned)(dir) + (unsigned)(stage) - 1u))
#define FFTMV_ALL_FP64 0x000u
#define FFTMV_MIXED_F 0x006u    /* F:  stages 2 (FFT) and 3 (SBGEMV) in FP32  */
#define FFTMV_MIXED_FADJ 0x180u /* F*: stages 3 (SBGEMV) and 4 (IFFT) in FP32 */
#define FFTMV_MIXED 0x186u      /* both of the above                          */
#define FFTMV_PREC_BITS 0x3FFu

/* ------------------------------------------------------------ plan flags
 * OR-ed into the mask argument of fftmv_setup (bits above the precision). */
/* Run the five stages as five kernels with materialised pad and unpad
 * buffers, instead of folding pad into the forward FFT's load and unpad into
 * the inverse FFT's store (same numbers, more memory traffic). */
#define FFTMV_FLAG_STAGED (1u << 16)
/* Keep Fhat in both complex64 and complex128 so that fftmv_set_mask can
 * switch to any precision mask without a new setup. */
#define FFTMV_FLAG_FHAT_BOTH (1u << 17)
#define FFTMV_FLAG_BITS (FFTMV_FLAG_STAGED | FFTMV_FLAG_FHAT_BOTH)

typedef struct fftmv_plan_s *fftmv_plan_t;

/* Build a plan: validate, allocate Fhat (complex64 if some SBGEMV stage is
 * FP32, complex128 if some SBGEMV stage is FP64; both with
 * FFTMV_FLAG_FHAT_BOTH), the twiddle tables and the workspace, then compute
 * Fhat_k for k = 0..Nt in FP64 on the device (batched real FFT of the Nd*Nm
 * zero-padded series of F) and round it once to each stored precision.
 * The frequency blocks are the precomputed operator of the page's five
 * stages (section 1.1): its error bound charges them with the roundoff of
 * a double-precision transform alone (the c_F eps_d term), which is why
 * they are computed in FP64 whatever the precision mask.
 * Returns after the stream has been synchronised.
 *   out     receives the plan; untouched on failure (nothing leaks)
 *   F_dev   device pointer, [Nt][Nd][Nm] FP64, read only, not retained
 *   mask    precision bits (FFTMV_PREC_BITS) | flags (FFTMV_FLAG_BITS)
 *   stream  stream for the setup work (0 = null stream) */
FFTMV_API int fftmv_setup(fftmv_plan_t *out, const double *F_dev, int64_t Nm, int64_t Nd, int64_t Nt,
                uint32_t mask, hipStream_t stream);

/* v = F m (section 1.1). m_dev [Nt][Nm] FP64 in, v_dev [Nt][Nd] FP64 out,
 * both device pointers; runs asynchronously on stream. */
FFTMV_API int fftmv_apply(fftmv_plan_t plan, const double *m_dev, double *v_dev, hipStream_t stream);

/* w = F* d with the conjugate-transpose frequency product (section 1.2).
 * d_dev [Nt][Nd] FP64 in, w_dev [Nt][Nm] FP64 out; asynchronous. */
FFTMV_API int fftmv_apply_adjoint(fftmv_plan_t plan, const double *d_dev, double *w_dev, hipStream_t stream);

/* For callers that cannot allocate device memory (code under stream
 * capture, serving loops, harnesses that forbid allocation): an apply of
 * direction dir (FFTMV_DIR_F: v = F m, as fftmv_apply; FFTMV_DIR_FADJ:
 * w = F* d, as fftmv_apply_adjoint) with the same kernels and the same
 * results, whose intermediate spectra and partial sums go to the library's
 * static device scratch instead of the plan's workspace. The scratch is one
 * fixed array of FFTMV_SCRATCH_BYTES per GPU, held from the library's first
 * use of a device until the process ends; the call allocates and frees
 * nothing. Layouts, alignment and ownership of in/out are those of
 * fftmv_apply / fftmv_apply_adjoint; asynchronous on stream.
 * Errors: FFTMV_ERR_INVALID_ARG as for the applies (and for dir not 0/1);
 * FFTMV_ERR_UNSUPPORTED_SIZE when the apply needs more than
 * FFTMV_SCRATCH_BYTES (the complex spectrum of the transformed side, e.g.
 * (Nt+1) x Nm complex64 for F in the mixed mask, plus the other side's, in
 * the precisions of the plan's mask); FFTMV_ERR_HIP if the scratch address
 * cannot be obtained. Every call on one GPU uses the same scratch, which
 * keeps the last call's contents: calls that overlap on one GPU (concurrent
 * streams, host threads) race and must be ordered by the caller. */
#define FFTMV_SCRATCH_BYTES (128u << 20)
FFTMV_API int fftmv_apply_scratch(fftmv_plan_t plan, int dir, const double *in, double *out, hipStream_t stream);

/* Free the plan's device memory. Synchronises the device first so that no
 * queued apply still uses it. NULL is accepted. */
FFTMV_API int fftmv_destroy(fftmv_plan_t plan);

/* Static string for a status code; never NULL. */
FFTMV_API const char *fftmv_status_string(int status);

/* Device bytes held by the plan: Fhat (all stored precisions) and the
 * workspace (stage buffers + twiddles). Either pointer may be NULL. */
FFTMV_API int fftmv_query(fftmv_plan_t plan, size_t *fhat_bytes, size_t *workspace_bytes);

/* Change the precision bits of a plan (flags are kept). Fails with
 * FFTMV_ERR_INVALID_ARG if the new mask needs an Fhat precision the plan did
 * not store. Must be ordered with the plan's applies like any other call on
 * the plan. */
FFTMV_API int fftmv_set_mask(fftmv_plan_t plan, uint32_t prec_mask);

/* Run stages first..last (1..5) of one direction, for stage-by-stage
 * checking. Stage s reads the buffer stage s-1 wrote (for s = 1, the FP64
 * input `in`) and writes its own buffer (for s = 5, the FP64 output `out`);
 * buffers are those of fftmv_buffer. Always runs the five-kernel form.
 * in/out may be NULL when first > 1 / last < 5. Asynchronous. */
FFTMV_API int fftmv_run_stages(fftmv_plan_t plan, int dir, int first, int last, const double *in, double *out,
                     hipStream_t stream);

/* Describe a plan-owned device buffer:
 *   which = 0: Fhat complex64, 1: Fhat complex128 -- [Nt+1][Nd][ld]
 *   which = 10 + 10*dir + s (s = 1..4): output buffer of stage s of
 *     direction dir -- stage 1: [Nt][ld] real (the nonzero half of the
 *     padded input; the zero half is never stored), stage 2 and 3:
 *     [Nt+1][ld] complex, stage 4: [Nt][ld] real.
 * ptr: device pointer (NULL if not allocated); ld: leading dimension in
 * elements; elem_bytes: 4/8 (real FP32/FP64) or 8/16 (complex64/128) --
 * buffers between two stages are stored in the narrower of the two stages'
 * precisions. Any out pointer may be NULL. */
FFTMV_API int fftmv_buffer(fftmv_plan_t plan, int which, void **ptr, int64_t *ld, int *elem_bytes);

/* ---------------------------------------------- precision selection
 * "Mixed-precision FFTMatvec performance optimization on AMD GPUs",
 * section 1.1, bounds the relative error of an apply by
 *
 *   kappa(Fhat) [ c1 e1 + (cF ed + c2 e2 + c4 e4) log2(Nt) + c3 e3 n
 *                 + c5 e5 log2(pc) ]
 *
 * where e_s is the unit roundoff of stage s (2^-24 in FP32, 2^-53 in FP64),
 * ed = 2^-53 that of the FP64 setup transform, n the length of the
 * SBGEMV's inner products and pc the number of processor columns of the
 * distributed form. Section 2.1 selects a configuration from an error
 * predictor (this bound), a performance predictor and a search of the
 * Pareto front of the candidates that meet the tolerance; section 2.2 runs
 * it over the 32 configurations (5 stages x 2 precisions) of a direction.
 *
 * The page prints no constants. Here they are parameters (defaults fitted
 * to measured errors), and these readings complete the bound:
 *   - n = Nm for F and Nd for F* (the inner length of each direction's
 *     SBGEMV); each direction has its own constants;
 *   - on one GPU pc = 1, where log2(pc) = 0 would make an FP32 stage 5
 *     free of error although it rounds the output once; the stage-5 term is
 *     taken as c5 e5 max(1, log2(pc)).
 * The performance predictor is a bandwidth model: each kernel of the apply
 * moves its algorithmic bytes through HBM at a sustained bandwidth B, each
 * batched FFT moves its tile through LDS once per radix pass (write and
 * read, Nt complex values per channel in the FFT stage's precision) at
 * B_lds, and each kernel adds a fixed time t0. Stage-boundary buffers hold
 * the narrower precision of their two stages, and the fused form (default)
 * folds stage 1 into the forward FFT's loads and stage 5 into the inverse
 * FFT's stores.
 *
 * Model parameters, FFTMV_MODEL_PARAMS doubles:
 *   [0..4] c1..c5   [5] cF   [6] B, [7] B_lds in bytes/s   [8] t0 in s
 * A configuration ("stage bits") is 5 bits for one direction, bit s-1 set
 * when stage s is FP32; its place in a plan mask is bits << (5*dir).
 * These functions are host-only and touch no device. */
#define FFTMV_MODEL_PARAMS 9

/* The library's default model parameters for direction dir (constants
 * fitted on one MI355X at Nm=5000, Nd=100, Nt=1000). */
FFTMV_API int fftmv_model_defaults(int dir, double *params);

/* Predicted relative error and apply time (seconds) of one configuration.
 *   flags   FFTMV_FLAG_STAGED selects the five-kernel byte model
 *   kappa   condition number of Fhat (fftmv_condition), >= 1
 *   params  FFTMV_MODEL_PARAMS values, or NULL for the defaults
 * Either output may be NULL. FFTMV_ERR_INVALID_ARG for sizes < 1, dir not
 * 0/1, stage_bits > 31, kappa < 1 or NaN, or parameters out of range
 * (negative constants, bandwidths <= 0); FFTMV_ERR_UNSUPPORTED_SIZE for an
 * Nt that fftmv_setup rejects. The same checks apply to the two calls
 * below. */
FFTMV_API int fftmv_predict(int64_t Nm, int64_t Nd, int64_t Nt, int dir, uint32_t stage_bits, uint32_t flags,
                            double kappa, const double *params, double *est_error, double *est_seconds);

/* Pareto front of the configurations of direction dir whose predicted
 * error is <= error_tol: no other feasible configuration is both faster and
 * more accurate. front[0..*count-1] (room for 32) is sorted by predicted
 * time, ties by error, then by fewer FP32 stages. *count = 0 when nothing is
 * feasible (the call still succeeds). */
FFTMV_API int fftmv_pareto_front(int64_t Nm, int64_t Nd, int64_t Nt, int dir, uint32_t flags, double kappa,
                                 double error_tol, const double *params, uint32_t *front, int *count);

/* select_precision(error_tol) of section 2.1: the fastest configuration on
 * the Pareto front. When no configuration meets the tolerance it returns
 * FFTMV_ERR_NO_CONFIG and reports the all-FP64 configuration (0) and its
 * prediction instead. Any output may be NULL. */
FFTMV_API int fftmv_select_precision(int64_t Nm, int64_t Nd, int64_t Nt, int dir, uint32_t flags, double kappa,
                                     double error_tol, const double *params, uint32_t *stage_bits,
                                     double *est_error, double *est_seconds);

/* kappa(Fhat), the condition number in the bound above: Fhat is block
 * diagonal, so kappa = max_k s_max(Fhat_k) / min_k s_min(Fhat_k) over the
 * min(Nd, Nm) singular values of each block (+Inf if some block is
 * singular). Estimated on the device by `iters` Lanczos steps (with full
 * reorthogonalisation) on each block's smaller Gram matrix, using the
 * plan's complex128 Fhat if it holds one, else its complex64 copy;
 * iters <= 0 picks min(n, 128), and iters is capped at min(n, 512) with
 * n = min(Nd, Nm). With iters >= n the values are those of the Gram
 * matrices up to rounding; with fewer, s_max is a lower and s_min an upper
 * bound (Ritz values), so kappa is under-estimated. Through the Gram matrix
 * s_min is resolved down to about sqrt(u) s_max (u the unit roundoff of
 * the Fhat copy used), so kappa is meaningful up to ~1e7 (complex128) or
 * ~1e3 (complex64 only).
 *   kappa      out, may be NULL
 *   sigma_max, sigma_min   out, host arrays of Nt+1 doubles (per
 *              frequency), may be NULL
 * Allocates and frees its own device workspace (~(iters+3) * (Nt+1) *
 * n * 16 bytes plus one long vector per frequency); synchronises `stream`
 * before returning. Must be ordered with the plan's applies. */
FFTMV_API int fftmv_condition(fftmv_plan_t plan, int iters, double *kappa, double *sigma_max, double *sigma_min,
                              hipStream_t stream);

/* Library version, (major << 16) | (minor << 8) | patch. */
FFTMV_API int fftmv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FFTMV_H */
