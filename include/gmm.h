/*
 * gmm.h - C ABI of libgmm: one fused Gaussian-mixture EM iteration on an
 * AMD Instinct MI355X (gfx950).
 *
 * What the library computes is defined by two pages:
 *   [LP-GMM]    the write-up on building a low-precision GMM operator
 *               (hotelren.com/news/5857197);
 *   [Flash-GMM] "Flash-GMM: a memory-efficient kernel for scalable soft
 *               clustering" (ai-feeds.com/i/paper/2606.10896).
 *
 * One EM iteration = gmm_em_step (E-step and M-step sufficient statistics in
 * one pass over X, without ever writing the N x K responsibility matrix)
 * followed by gmm_finalize (new parameters from the statistics).  The
 * parameters must first be loaded with gmm_prepare.  gmm_loglik is the E-step
 * alone ([LP-GMM] 1.1: inference needs only the E-step).
 *
 * Conventions for every call:
 *  - All data pointers are DEVICE pointers unless the comment says "host".
 *    The caller owns every buffer (X, parameters, outputs and the workspace)
 *    and the stream; the library never allocates device or host memory.
 *  - Calls are asynchronous and stream-ordered on `stream` (0 = the null
 *    stream); they return before the GPU work finishes.  Argument errors are
 *    detected on the host and returned before anything is launched.
 *  - Floating-point parameters are fp32 row-major arrays:
 *      pi  [K]; mu [K*D];
 *      cov [K*D] (GMM_COV_DIAG, variances), [K] (GMM_COV_ISO, one variance
 *          per component), [K*D*D] (GMM_COV_FULL, covariance matrices).
 *  - X is row-major [N rows, row stride ldx elements], stored as fp32, bf16
 *    or fp16 (gmm_desc.x_dtype).  The vectorised loaders are used when X is
 *    16-byte aligned, ldx*elem_size is a multiple of 16 and D is a multiple
 *    of 16/elem_size; any other layout takes a slower element-wise loader.
 *  - exp, log, the normalising sums and every statistic are fp32 or wider
 *    whatever the storage type ([LP-GMM] 1.3 first boundary, 2.1).
 *  - One workspace serves one descriptor; concurrent calls on the same
 *    workspace race.  Results are bitwise reproducible for a given device,
 *    descriptor and input.
 */
#ifndef GMM_H
#define GMM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GMM_OK = 0,
    GMM_E_ARG = 1,          /* null pointer, bad size, bad enum, bad alignment */
    GMM_E_UNSUPPORTED = 2,  /* (cov, dtype, D, K) combination not provided.
                               Provided: D <= 128 throughout; diagonal with
                               K <= 64 (any storage type); diagonal or
                               isotropic with bf16 / fp16 storage, K <= 4096;
                               full covariance with fp16 storage, K <= 256 */
    GMM_E_WORKSPACE = 3,    /* ws_bytes smaller than gmm_workspace_bytes() */
    GMM_E_HIP = 4,          /* a HIP runtime call or kernel launch failed */
    GMM_E_NOT_PD = 5,       /* reported by gmm_diagnostics only */
    GMM_E_NONFINITE = 6     /* reported by gmm_diagnostics only */
} gmm_status;

typedef enum { GMM_COV_DIAG = 0, GMM_COV_ISO = 1, GMM_COV_FULL = 2 } gmm_cov;
typedef enum { GMM_F32 = 0, GMM_BF16 = 1, GMM_F16 = 2 } gmm_dtype;

/* Problem description ([Flash-GMM] Method, inputs: X in R^{N x D}, K
 * components and the covariance type are the only configuration).  */
typedef struct {
    int64_t n;          /* points N >= 0 (gmm_em_step needs N >= 1) */
    int64_t d;          /* dimensions D >= 1 */
    int64_t k;          /* components K >= 1 */
    int64_t ldx;        /* row stride of X in elements, >= d */
    int32_t cov;        /* gmm_cov */
    int32_t x_dtype;    /* gmm_dtype: storage type of X */
    float var_floor;    /* variances are clamped below at this (>= 0); 1e-6 */
    float ridge_rel;    /* GMM_COV_FULL: eps = ridge_rel*|trace(C)|/D is added
                           to the diagonal before the Cholesky factorisation
                           ([LP-GMM] 4.1); 1e-3 */
} gmm_desc;

/* Device-side health report, filled by gmm_diagnostics: the flags that
 * [LP-GMM] 3.3 asks the preprocessing to raise (an indefinite covariance is
 * detected and marked there, never branched on in the hot loop), the
 * failure modes of 4.1 (not positive definite) and 4.2 (underflow to 0/0 =
 * NaN), and the checks of the debugging order in 5.1 (weights, non-finite
 * values, small variances that make the fp16 score swing). */
typedef struct {
    int32_t bad_params;      /* components whose prepared variance/covariance
                                was non-positive or non-finite */
    int32_t not_pd;          /* full covariance: components still indefinite
                                after the ridge retries (their weight is
                                treated as 0) */
    int32_t ridge_retries;   /* full covariance: largest escalation count */
    int32_t empty;           /* components with s0 < 1e-6 at the last finalize */
    int32_t nonfinite;       /* 1 if the last LL or statistics were NaN/Inf */
    int32_t x_range;         /* large-K (fp16 operand) plans: 1 if the last
                                pass met a value of X whose scaled square
                                exceeded the fp16 range (the centre and scale
                                come from a sample of X).  The pass then fails
                                visibly: its LL is NaN, nonfinite is set and
                                gmm_finalize keeps theta.  NaN in X shows up as
                                a non-finite LL */
    int32_t ill_cond;        /* components whose expanded score [y^2, y, 1] .
                                panel is estimated to carry more than 1 nat of
                                rounding error near their own mean (a variance
                                small against the component's distance from
                                the data centre, [LP-GMM] 5.1 fourth step).
                                Large-K plans (fp16 panel): they are taken out
                                of the panel and scored in the exact centred
                                form in fp32 ([LP-GMM] 1.2, 1.3), so the count
                                is informational.  Diagonal fp32 plans (split
                                fp16 panel, about 22 bits): counted from the
                                prepared theta; only components near the
                                variance floor far from the centre get there,
                                and their LL contribution then carries that
                                error (their statistics do not).  0 for full
                                covariance, whose score is centred */
    int32_t reserved;
    double  ll;              /* LL of the last gmm_em_step / gmm_loglik */
} gmm_diag;

/* Bytes of device workspace the descriptor needs (host call, no GPU work).
 * The size is O(K*D^2 + P*K*D + N*G) for a fixed number P of partial slots,
 * where G is 1 for the diagonal K <= 64 plans and the number of component
 * slices (K / 256, large-K plans) or groups (K / 16 when K > 16 or D > 64,
 * full covariance) whose per-point log-sum-exp is kept between two passes;
 * it never holds the N x K responsibility matrix ([Flash-GMM] key insight:
 * memory O(N + K) per slice).
 * Returns GMM_E_ARG / GMM_E_UNSUPPORTED for descriptors the library rejects. */
gmm_status gmm_workspace_bytes(const gmm_desc* desc, size_t* bytes /* host */);

/* Load parameters theta = (pi, mu, cov) and precompute per-component
 * quantities ([LP-GMM] 3.1, Preprocess kernel): log-normaliser, precisions
 * and the score panel; for full covariance the ridged Cholesky factor L and
 * its inverse, which the E-step applies to x - mu in place of the forward
 * solve ([LP-GMM] 1.2 route 2, 4.1).  pi/mu/cov are device fp32; they are copied,
 * so the caller may reuse them after the call is stream-ordered. */
gmm_status gmm_prepare(const gmm_desc* desc, void* ws, size_t ws_bytes,
                       const float* pi, const float* mu, const float* cov,
                       hipStream_t stream);

/* E-step + M-step sufficient statistics in one pass over X ([Flash-GMM]
 * Method, fused E-M step: per tile, Mahalanobis terms and the softmax over K
 * in registers, then s0 = sum gamma, s1 = sum gamma x, s2 = sum gamma x^2 /
 * sum gamma |x|^2 / sum gamma x x^T accumulated on chip).  The statistics
 * stay in the workspace.  ll_out (device double, nullable) receives
 * LL(theta) = sum_n log sum_k pi_k N(x_n | theta_k), natural log, under the
 * prepared parameters.  Needs N >= 1. */
gmm_status gmm_em_step(const gmm_desc* desc, void* ws, size_t ws_bytes,
                       const void* x, double* ll_out, hipStream_t stream);

/* M-step ([Flash-GMM] Method, parameter update): pi' = s0/N,
 * mu' = s1/s0, variance' = max(s2/s0 - mu'^2, var_floor) (diag; iso divides
 * the trace by D; full: s2/s0 - mu' mu'^T).  A component with s0 < 1e-6
 * keeps its mean and covariance and gets pi' = s0/N.  Writes theta' (device
 * fp32, same layouts as gmm_prepare; any of the three may be NULL) AND
 * prepares the workspace for theta', so the next gmm_em_step can follow
 * directly without gmm_prepare. */
gmm_status gmm_finalize(const gmm_desc* desc, void* ws, size_t ws_bytes,
                        float* pi_out, float* mu_out, float* cov_out,
                        hipStream_t stream);

/* E-step only ([LP-GMM] 1.1) under the prepared parameters.  ll_out (device
 * double, nullable) gets sum_n lse_n; point_lse (device fp32 [N], nullable)
 * gets lse_n = log sum_k pi_k N(x_n | theta_k); point_argmax (device int32
 * [N], nullable) gets argmax_k of the responsibility (lowest k on ties).
 * N = 0 is allowed (LL = 0). */
gmm_status gmm_loglik(const gmm_desc* desc, void* ws, size_t ws_bytes,
                      const void* x, double* ll_out, float* point_lse,
                      int32_t* point_argmax, hipStream_t stream);

/* Largest m of gmm_assign. */
#define GMM_MAX_TOPM 16

/* Top-m soft assignment under the prepared parameters (E-step only).
 * [Flash-GMM] Key findings: the soft responsibilities let a point near a
 * cluster boundary belong to several clusters; Deployment: the coarse
 * quantiser of an IVF index assigns each vector to several lists.  For every
 * point n the m components with the largest responsibility gamma_nk, in
 * decreasing order (ties: the lower component index first), are written to
 * out_idx[n*m + i] (device int32) and gamma_nk to out_gamma[n*m + i] (device
 * fp32).  Components with log-joint -inf (zero weight) are never listed:
 * columns past the listed components hold index -1 and 0.  1 <= m <=
 * GMM_MAX_TOPM, else GMM_E_ARG.  ll_out (device double, nullable) gets the LL
 * as gmm_loglik does.  N = 0 is allowed.  Large-K plans: the outputs also
 * carry intermediate values between the passes over X of one call. */
gmm_status gmm_assign(const gmm_desc* desc, void* ws, size_t ws_bytes, const void* x,
                      int32_t m, int32_t* out_idx, float* out_gamma, double* ll_out,
                      hipStream_t stream);

/* Start of gmm_fit. */
typedef enum {
    GMM_INIT_GIVEN = 0,          /* theta_0 is read from pi / mu / cov */
    GMM_INIT_RANDOM_POINTS = 1   /* K distinct rows of X (seeded) as means, unit
                                    (co)variances, weights 1/K; needs K <= N */
} gmm_init;

typedef struct {
    int32_t max_iter;   /* iterations at most, >= 1 */
    int32_t init;       /* gmm_init */
    uint64_t seed;      /* GMM_INIT_RANDOM_POINTS: generator state */
    double tol;         /* stop after iteration t >= 1 once |LL_t - LL_t-1| / N < tol
                           (0: run max_iter iterations) */
    int32_t batch;      /* iterations launched between two host checks, >= 1 */
    int32_t use_graph;  /* 1: capture one iteration into a HIP graph and replay it
                           (needs a non-null stream) */
} gmm_fit_opts;

/* EM iterations to convergence ([Flash-GMM] Method, outputs: the fused step is
 * called repeatedly until the log-likelihood converges; [LP-GMM] 1.1:
 * training alternates E and M steps).  Iteration t = gmm_em_step (LL_t under
 * theta_t) + gmm_finalize (theta_t+1); the loop stops after iteration t once
 * t >= 1 and |LL_t - LL_t-1| / N < tol, after max_iter iterations, or on a
 * non-finite LL (theta_t+1 is then not taken).  The device decides and
 * records; the host synchronises once per `batch` iterations.
 * GMM_INIT_RANDOM_POINTS draws K distinct rows with Floyd's K-subset
 * algorithm (Bentley and Floyd, CACM 1987) from SplitMix64 (Steele, Lea and
 * Flood, OOPSLA 2014) seeded with opts->seed, the draw in [0, j] being the
 * output modulo j + 1, and writes that start into pi / mu / cov.
 * pi / mu / cov: device fp32, in: theta_0 (GMM_INIT_GIVEN), out: the final
 * theta.  ll_hist: device double [max_iter] (nullable), LL_t per iteration.
 * n_iter: host (nullable), iterations taken.  Synchronous: returns after the
 * loop, with the workspace prepared for the final theta.  Creates and
 * destroys a HIP graph when use_graph is set; allocates no memory itself. */
gmm_status gmm_fit(const gmm_desc* desc, void* ws, size_t ws_bytes, const void* x,
                   const gmm_fit_opts* opts, float* pi, float* mu, float* cov,
                   double* ll_hist, int32_t* n_iter, hipStream_t stream);

/* Copy the sufficient statistics of the last EM iteration into device fp64
 * buffers (each nullable): s0 [K]; s1 [K*D]; s2 [K*D] (diag: sum gamma x^2),
 * [K] (iso: sum gamma |x|^2) or [K*D*D] (full: sum gamma x x^T) - the
 * zeroth, first and second moments of [Flash-GMM] Method (statistics
 * accumulated on chip tile by tile), in raw units of x.  The per-workgroup
 * partials of gmm_em_step are reduced by gmm_finalize ([LP-GMM] 3.1, M-step:
 * partial reductions per block, then a global one), so call this after
 * gmm_finalize; the values are those of the em_step it finished.  Errors:
 * GMM_E_ARG for a null descriptor or workspace, GMM_E_WORKSPACE,
 * GMM_E_HIP if a copy fails. */
gmm_status gmm_get_stats(const gmm_desc* desc, const void* ws, size_t ws_bytes,
                         double* s0, double* s1, double* s2, hipStream_t stream);

/* Synchronises `stream` and copies the device health flags to *out (host). */
gmm_status gmm_diagnostics(const gmm_desc* desc, const void* ws, size_t ws_bytes,
                           gmm_diag* out /* host */, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): one EM
 * iteration, gmm_prepare(pi, mu, cov) + gmm_em_step(x) + gmm_finalize, with no
 * workspace argument and no allocation.  The workspace is a fixed device
 * array of gmm_noalloc_max_workspace() bytes (128 MiB) inside the library,
 * one copy per device, held until the process ends; a descriptor whose
 * gmm_workspace_bytes exceeds it returns GMM_E_WORKSPACE before anything is
 * launched.  All calls on one device share that array: calls that overlap on
 * a device race (serialise them, e.g. on one stream).  Arguments as in
 * gmm_prepare / gmm_em_step / gmm_finalize (ll_out and the three outputs
 * nullable); the results equal those of that sequence on a caller workspace. */
gmm_status gmm_em_iteration_noalloc(const gmm_desc* desc, const float* pi, const float* mu,
                                    const float* cov, const void* x, double* ll_out,
                                    float* pi_out, float* mu_out, float* cov_out,
                                    hipStream_t stream);

/* Bytes of the internal workspace of gmm_em_iteration_noalloc. */
size_t gmm_noalloc_max_workspace(void);

/* Static string for a status code. */
const char* gmm_status_str(gmm_status status);

/* Library version, "major.minor.patch". */
const char* gmm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GMM_H */
