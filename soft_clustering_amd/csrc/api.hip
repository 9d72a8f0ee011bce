// C ABI of libgmm (declared in include/gmm.h): argument validation, the
// workspace layout and dispatch to the kernel families.  The library never
// allocates memory; every launch goes to the caller's stream.

#include <math.h>
#include <stdlib.h>
#include <string.h>

#include "common.h"
#include "diag_internal.h"
#include "full_internal.h"
#include "largek_internal.h"

namespace gmm {

bool diag_shape_supported(int dp, int kb);

int device_cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        cached[dev] = cus;
    }
    return cached[dev];
}

// Tuning: GMM_SEGMENT_TILES (environment, positive integer) overrides the
// length of the fp32 accumulation runs of the statistics passes (tiles per
// workgroup or wave and launch segment); unset or invalid: each family's
// default.  Read at every call, so a process can change it between calls.
static int64_t segment_tiles_override() {
    const char* v = getenv("GMM_SEGMENT_TILES");
    if (v == nullptr || *v == 0) return 0;
    char* end = nullptr;
    const long long t = strtoll(v, &end, 10);
    if (end == v || *end != 0 || t < 1 || t > ((int64_t)1 << 40)) return 0;
    return (int64_t)t;
}

static int pad_dim(int64_t d) {
    if (d <= 16) return 16;
    if (d <= 32) return 32;
    if (d <= 64) return 64;
    if (d <= 128) return 128;
    return -1;
}

gmm_status make_plan(const gmm_desc* desc, Plan* p) {
    if (desc == nullptr || p == nullptr) return GMM_E_ARG;
    memset(p, 0, sizeof(*p));
    p->n = desc->n;
    p->d = desc->d;
    p->k = desc->k;
    p->ldx = desc->ldx;
    p->cov = desc->cov;
    p->xdt = desc->x_dtype;
    p->var_floor = desc->var_floor;
    p->ridge_rel = desc->ridge_rel;
    if (p->n < 0 || p->d < 1 || p->k < 1 || p->ldx < p->d) return GMM_E_ARG;
    if (p->n > ((int64_t)1 << 40) || p->d > (1 << 20) || p->k > (1 << 20)) return GMM_E_ARG;
    if (p->ldx > ((int64_t)1 << 22)) return GMM_E_ARG;   // tile offsets are 32-bit
    if (p->cov < GMM_COV_DIAG || p->cov > GMM_COV_FULL) return GMM_E_ARG;
    if (p->xdt < GMM_F32 || p->xdt > GMM_F16) return GMM_E_ARG;
    if (!(p->var_floor >= 0.0f) || !isfinite(p->var_floor)) return GMM_E_ARG;
    if (!(p->ridge_rel >= 0.0f) || !isfinite(p->ridge_rel)) return GMM_E_ARG;
    p->seg_tiles = segment_tiles_override();

    const size_t A = 256;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = align_up(off + bytes, A);
        return o;
    };

    const int64_t kb64 = (p->k + 15) / 16;
    const bool x16 = p->xdt == GMM_BF16 || p->xdt == GMM_F16;
    if (p->cov == GMM_COV_DIAG && kb64 <= 4) {
        const int dp = pad_dim(p->d);
        const int kb = (int)kb64;
        if (dp < 0 || !diag_shape_supported(dp, kb)) return GMM_E_UNSUPPORTED;
        p->path = PATH_DIAG_F32;
        p->dp = dp;
        p->kb = kb;
        p->p_max = 512;   // one workgroup per CU on up to 512 CUs
        p->ncols = 1 + 2 * p->d;
        p->off_pi = take(sizeof(float) * p->k);
        p->off_mu = take(sizeof(float) * p->k * p->d);
        p->off_cov = take(sizeof(float) * p->k * p->d);
        p->off_shift = take(sizeof(float) * 2 * dp);
        p->off_panel = take(sizeof(float) * (dp / 4) * 2 * kb * 64);
        p->off_part = take(sizeof(double) * p->p_max * p->k * p->ncols);
        p->off_part_ll = take(sizeof(double) * p->p_max);
        p->off_stats = take(sizeof(double) * p->k * p->ncols);
        p->off_ll = take(sizeof(double));
        p->off_diag = take(sizeof(int) * (2 * p->k + 2));
        p->off_chunk = take(sizeof(double) * 4 * p->k * diag_chunks(*p));
        p->off_ctl = take(fit_ctl_bytes(*p));
        p->total = off;
        return GMM_OK;
    }
    if ((p->cov == GMM_COV_DIAG || p->cov == GMM_COV_ISO) && x16) {
        // large-K family: fp16 MFMA operands, 256-component slices
        int dp = pad_dim(p->d);
        if (dp < 0 || p->k > 16 * kLkSlice) return GMM_E_UNSUPPORTED;
        if (dp < 32) dp = 32;
        const bool iso = p->cov == GMM_COV_ISO;
        const int S = (int)((p->k + kLkSlice - 1) / kLkSlice);
        const int64_t tiles = (p->n + kLkT - 1) / kLkT;
        p->path = PATH_LARGEK;
        p->dp = dp;
        p->kb = (int)kb64;
        p->lk_slices = S;
        p->lk_kpad = S * kLkSlice;
        // one workgroup per CU on up to 256 CUs, never more than S per tile
        int64_t pm = 256;
        if (pm > S * (tiles < 1 ? 1 : tiles)) pm = S * (tiles < 1 ? 1 : tiles);
        p->p_max = (int)pm;
        p->ncols = lk_ncols(p->cov, p->d);
        p->off_pi = take(sizeof(float) * p->k);
        p->off_mu = take(sizeof(float) * p->k * p->d);
        p->off_cov = take(sizeof(float) * p->k * (iso ? 1 : p->d));
        p->off_shift = take(sizeof(float) * (2 + 3 * kLkScanWgs) * dp);
        // panel: (features + 16 bias slots) / 16 MFMA steps x Kpad / 32 blocks x 64 lanes x 16 B
        p->off_panel = take((size_t)(((iso ? 1 : 2) * dp + 16) / 16) * (p->lk_kpad / 32) * 64 * 16);
        p->off_chunk = take(sizeof(float) * (2 * p->lk_kpad + 4));   // kmax, prm, c0
        // per-(slice, point) LSE, argmax and maximum, and a row for the exactly
        // scored components: the two sweeps, top-m assignment
        p->off_lse = take(sizeof(float) * (size_t)(S + 1) * p->n);
        p->off_arg = take((sizeof(int) + sizeof(float)) * (size_t)(S + 1) * p->n);
        p->off_xc = take(sizeof(int) * (2 * p->k + 16));
        p->off_xcpart = take(lk_xc_part_bytes(p->k, lk_ncols(p->cov, p->d)));
        p->off_part = take(sizeof(double) * (size_t)p->p_max * kLkSlice * p->ncols);
        p->off_part_ll = take((sizeof(double) + sizeof(int)) * kLkLLSlots);
        p->off_stats = take(sizeof(double) * p->k * p->ncols);
        p->off_ll = take(sizeof(double));
        p->off_diag = take(sizeof(int) * (2 * p->k + 4));
        p->off_ctl = take(fit_ctl_bytes(*p));
        p->total = off;
        return GMM_OK;
    }
    if (p->cov == GMM_COV_FULL && p->xdt == GMM_F16) {
        // full covariance: fp16 X, split fp16 whitening panel, fp16 MFMA whitening and moments
        if (p->d > 128 || p->k > kFullMaxK) return GMM_E_UNSUPPORTED;
        int dp = pad_dim(p->d);
        const int64_t tiles = (p->n + kFullT - 1) / kFullT;
        const int G = full_groups(p->k);          // groups of 16 components
        const int64_t kpad = (int64_t)kFullKP * G;
        p->path = PATH_FULL;
        p->dp = dp;
        p->kb = G;
        p->p_max = (int)(tiles < 1 ? 1 : (tiles > 256 ? 256 : tiles));
        p->ncols = 1 + p->d + p->d * p->d;
        const int64_t ncolp = full_ncolp(p->d);
        p->off_pi = take(sizeof(float) * p->k);
        p->off_mu = take(sizeof(float) * p->k * p->d);
        p->off_cov = take(sizeof(float) * p->k * p->d * p->d);
        p->off_panel = take(sizeof(uint4) * full_w_vecs(dp) * G);
        p->off_shift = take(sizeof(float) * (kpad * full_dpo(dp) + kpad * dp + 2 * kpad));
        if (full_lse_pass(p->k, dp)) {   // per-(group, point) LSE, argmax and maximum
            p->off_lse = take(sizeof(float) * (size_t)G * p->n);
            p->off_arg = take((sizeof(int) + sizeof(float)) * (size_t)G * p->n);
        }
        p->off_part = take(sizeof(float) * (size_t)G * p->p_max * kFullKP * ncolp);
        p->off_part_ll = take(sizeof(double) * kFullLLSlots);
        p->off_chunk = take(sizeof(double) * p->k * ncolp);
        p->off_stats = take(sizeof(double) * p->k * p->ncols);
        p->off_ll = take(sizeof(double));
        p->off_diag = take(sizeof(int) * (2 * p->k + 4));
        p->off_ctl = take(fit_ctl_bytes(*p));
        p->total = off;
        return GMM_OK;
    }
    return GMM_E_UNSUPPORTED;
}

static gmm_status check_ws(const Plan& p, const void* ws, size_t ws_bytes) {
    if (ws == nullptr) return GMM_E_ARG;
    if ((uintptr_t)ws % 256 != 0) return GMM_E_ARG;
    if (ws_bytes < p.total) return GMM_E_WORKSPACE;
    return GMM_OK;
}

}  // namespace gmm

using namespace gmm;

extern "C" {

gmm_status gmm_workspace_bytes(const gmm_desc* desc, size_t* bytes) {
    if (bytes == nullptr) return GMM_E_ARG;
    Plan p;
    gmm_status st = make_plan(desc, &p);
    if (st != GMM_OK) return st;
    *bytes = p.total;
    return GMM_OK;
}

gmm_status gmm_prepare(const gmm_desc* desc, void* ws, size_t ws_bytes, const float* pi,
                       const float* mu, const float* cov, hipStream_t stream) {
    Plan p;
    gmm_status st = make_plan(desc, &p);
    if (st != GMM_OK) return st;
    if ((st = check_ws(p, ws, ws_bytes)) != GMM_OK) return st;
    if (pi == nullptr || mu == nullptr || cov == nullptr) return GMM_E_ARG;
    if (p.path == PATH_LARGEK) return lk_prepare(p, (char*)ws, pi, mu, cov, stream);
    if (p.path == PATH_FULL) return full_prepare(p, (char*)ws, pi, mu, cov, stream);
    return diag_prepare(p, (char*)ws, pi, mu, cov, stream);
}

gmm_status gmm_em_step(const gmm_desc* desc, void* ws, size_t ws_bytes, const void* x,
                       double* ll_out, hipStream_t stream) {
    Plan p;
    gmm_status st = make_plan(desc, &p);
    if (st != GMM_OK) return st;
    if ((st = check_ws(p, ws, ws_bytes)) != GMM_OK) return st;
    if (x == nullptr || p.n < 1) return GMM_E_ARG;
    if (p.path == PATH_LARGEK) return lk_em_step(p, (char*)ws, x, ll_out, stream);
    if (p.path == PATH_FULL) return full_em_step(p, (char*)ws, x, ll_out, stream);
    return diag_em_step(p, (char*)ws, x, ll_out, stream);
}

gmm_status gmm_finalize(const gmm_desc* desc, void* ws, size_t ws_bytes, float* pi_out,
                        float* mu_out, float* cov_out, hipStream_t stream) {
    Plan p;
    gmm_status st = make_plan(desc, &p);
    if (st != GMM_OK) return st;
    if ((st = check_ws(p, ws, ws_bytes)) != GMM_OK) return st;
    if (p.n < 1) return GMM_E_ARG;
    if (p.path == PATH_LARGEK) return lk_finalize(p, (char*)ws, pi_out, mu_out, cov_out, stream);
    if (p.path == PATH_FULL) return full_finalize(p, (char*)ws, pi_out, mu_out, cov_out, stream);
    return diag_finalize(p, (char*)ws, pi_out, mu_out, cov_out, stream);
}

gmm_status gmm_loglik(const gmm_desc* desc, void* ws, size_t ws_bytes, const void* x,
                      double* ll_out, float* point_lse, int32_t* point_argmax,
                      hipStream_t stream) {
    Plan p;
    gmm_status st = make_plan(desc, &p);
    if (st != GMM_OK) return st;
    if ((st = check_ws(p, ws, ws_bytes)) != GMM_OK) return st;
    if (x == nullptr && p.n > 0) return GMM_E_ARG;
    if (p.path == PATH_LARGEK)
        return lk_loglik(p, (char*)ws, x, ll_out, point_lse, point_argmax, stream);
    if (p.path == PATH_FULL)
        return full_loglik(p, (char*)ws, x, ll_out, point_lse, point_argmax, stream);
    return diag_loglik(p, (char*)ws, x, ll_out, point_lse, point_argmax, stream);
}

gmm_status gmm_assign(const gmm_desc* desc, void* ws, size_t ws_bytes, const void* x, int32_t m,
                      int32_t* out_idx, float* out_gamma, double* ll_out, hipStream_t stream) {
    Plan p;
    gmm_status st = make_plan(desc, &p);
    if (st != GMM_OK) return st;
    if ((st = check_ws(p, ws, ws_bytes)) != GMM_OK) return st;
    if (m < 1 || m > GMM_MAX_TOPM) return GMM_E_ARG;
    if (p.n > 0 && (x == nullptr || out_idx == nullptr || out_gamma == nullptr)) return GMM_E_ARG;
    if (p.path == PATH_LARGEK) return lk_assign(p, (char*)ws, x, m, out_idx, out_gamma, ll_out, stream);
    if (p.path == PATH_FULL) return full_assign(p, (char*)ws, x, m, out_idx, out_gamma, ll_out, stream);
    return diag_assign(p, (char*)ws, x, m, out_idx, out_gamma, ll_out, stream);
}

gmm_status gmm_get_stats(const gmm_desc* desc, const void* ws, size_t ws_bytes, double* s0,
                         double* s1, double* s2, hipStream_t stream) {
    Plan p;
    gmm_status st = make_plan(desc, &p);
    if (st != GMM_OK) return st;
    if ((st = check_ws(p, ws, ws_bytes)) != GMM_OK) return st;
    const char* base = (const char*)ws + p.off_stats;
    const size_t pitch = sizeof(double) * p.ncols;
    hipError_t e = hipSuccess;
    if (s0 && e == hipSuccess)
        e = hipMemcpy2DAsync(s0, sizeof(double), base, pitch, sizeof(double), p.k,
                             hipMemcpyDeviceToDevice, stream);
    if (s1 && e == hipSuccess)
        e = hipMemcpy2DAsync(s1, sizeof(double) * p.d, base + sizeof(double), pitch,
                             sizeof(double) * p.d, p.k, hipMemcpyDeviceToDevice, stream);
    // diag: sum gamma x^2 [D]; iso: sum gamma |x|^2 [1]; full: sum gamma x x^T [D*D]
    const int64_t w2 = p.cov == GMM_COV_ISO ? 1 : (p.cov == GMM_COV_FULL ? p.d * p.d : p.d);
    if (s2 && e == hipSuccess)
        e = hipMemcpy2DAsync(s2, sizeof(double) * w2, base + sizeof(double) * (1 + p.d), pitch,
                             sizeof(double) * w2, p.k, hipMemcpyDeviceToDevice, stream);
    return e == hipSuccess ? GMM_OK : GMM_E_HIP;
}

// Diagonal fp32 path: components whose split-fp16 expanded score [y^2 | y] .
// panel (about 22 significant bits per term) is estimated to carry more than
// one nat of rounding error near their own mean: the terms A y^2 and B y at
// |mu - c| + 3 sigma from the centre c, relative error 2^-22 each, random
// signs ([LP-GMM] 5.1 fourth step: a small variance makes the score swing).
// A component at the variance floor far from the centre reaches tens of nats
// (the LL then misses the fp32 bar; the statistics keep it, since such a
// component owns its points whatever the error).  Host arithmetic on theta
// and the centre, read in fixed-size pieces.
static hipError_t diag_ill_cond(const Plan& p, const char* base, int32_t* count) {
    constexpr int kCompPiece = 16, kMaxD = 128;
    float cen[kMaxD], mu[kCompPiece * kMaxD], var[kCompPiece * kMaxD];
    const int d = (int)p.d;
    hipError_t e = hipMemcpy(cen, base + p.off_shift, sizeof(float) * d, hipMemcpyDeviceToHost);
    int cnt = 0;
    for (int64_t k0 = 0; k0 < p.k && e == hipSuccess; k0 += kCompPiece) {
        const int m = (int)(p.k - k0 < kCompPiece ? p.k - k0 : kCompPiece);
        e = hipMemcpy(mu, base + p.off_mu + sizeof(float) * k0 * d, sizeof(float) * m * d,
                      hipMemcpyDeviceToHost);
        if (e == hipSuccess)
            e = hipMemcpy(var, base + p.off_cov + sizeof(float) * k0 * d, sizeof(float) * m * d,
                          hipMemcpyDeviceToHost);
        for (int i = 0; i < m && e == hipSuccess; ++i) {
            double err2 = 0.0;
            bool ok = true;
            for (int dd = 0; dd < d; ++dd) {
                const double v = var[i * d + dd], mc = fabs((double)mu[i * d + dd] - (double)cen[dd]);
                if (!(v > 0.0) || !isfinite(v) || !isfinite(mc)) {
                    ok = false;
                    break;
                }
                const double yt = mc + 3.0 * sqrt(v);
                const double ta = 0.5 * kLog2e * yt * yt / v, tb = kLog2e * mc * yt / v;
                err2 += ta * ta + tb * tb;
            }
            const double nats = sqrt(err2) * ldexp(1.0, -22) * 0.81649658 * 0.69314718;
            if (ok && nats > 1.0) ++cnt;
        }
    }
    *count = cnt;
    return e;
}

gmm_status gmm_diagnostics(const gmm_desc* desc, const void* ws, size_t ws_bytes, gmm_diag* out,
                           hipStream_t stream) {
    Plan p;
    gmm_status st = make_plan(desc, &p);
    if (st != GMM_OK) return st;
    if ((st = check_ws(p, ws, ws_bytes)) != GMM_OK) return st;
    if (out == nullptr) return GMM_E_ARG;
    if (hipStreamSynchronize(stream) != hipSuccess) return GMM_E_HIP;
    // The flags are read in fixed-size pieces into stack buffers, so this
    // call allocates nothing whatever K is.
    constexpr int kPiece = 256;
    int fl[kPiece], rt[kPiece], misc[2];
    double ck[kPiece * 4];
    const char* base = (const char*)ws;
    const int* dflags = (const int*)(base + p.off_diag);
    double ll = 0.0;
    hipError_t e = hipMemcpy(&ll, base + p.off_ll, sizeof(double), hipMemcpyDeviceToHost);
    if (e == hipSuccess)
        e = hipMemcpy(misc, dflags + 2 * p.k, sizeof(misc), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return GMM_E_HIP;
    memset(out, 0, sizeof(*out));
    // diagonal fp32 path: per-(component, chunk) counts of bad / non-finite values
    const bool dg = p.path == PATH_DIAG_F32;
    const int nch = dg ? diag_chunks(p) : 0;
    const double* dchunk = (const double*)(base + p.off_chunk);
    for (int64_t k0 = 0; k0 < p.k && e == hipSuccess; k0 += kPiece) {
        const int m = (int)(p.k - k0 < kPiece ? p.k - k0 : kPiece);
        e = hipMemcpy(fl, dflags + k0, sizeof(int) * m, hipMemcpyDeviceToHost);
        if (e == hipSuccess)
            e = hipMemcpy(rt, dflags + p.k + k0, sizeof(int) * m, hipMemcpyDeviceToHost);
        for (int i = 0; i < m && e == hipSuccess; ++i) {
            int f = fl[i];
            for (int c0 = 0; c0 < nch && e == hipSuccess; c0 += kPiece) {
                const int mc = nch - c0 < kPiece ? nch - c0 : kPiece;
                e = hipMemcpy(ck, dchunk + ((k0 + i) * nch + c0) * 4, sizeof(double) * 4 * mc,
                              hipMemcpyDeviceToHost);
                for (int c = 0; c < mc; ++c) {
                    if (ck[4 * c + 2] > 0.0) f |= 1;
                    if (ck[4 * c + 3] > 0.0) f |= 8;
                }
            }
            if (f & 1) out->bad_params++;
            if (f & 2) out->not_pd++;
            if (f & 4) out->empty++;
            if (f & 8) out->nonfinite = 1;
            if (f & 16) out->ill_cond++;
            if (rt[i] > out->ridge_retries) out->ridge_retries = rt[i];
        }
    }
    if (misc[0]) out->nonfinite = 1;
    if (p.path == PATH_LARGEK) out->x_range = misc[1];
    if (dg && e == hipSuccess) e = diag_ill_cond(p, base, &out->ill_cond);
    out->ll = ll;
    return e == hipSuccess ? GMM_OK : GMM_E_HIP;
}

const char* gmm_status_str(gmm_status s) {
    switch (s) {
        case GMM_OK: return "ok";
        case GMM_E_ARG: return "invalid argument";
        case GMM_E_UNSUPPORTED: return "unsupported (covariance, dtype, D, K) combination";
        case GMM_E_WORKSPACE: return "workspace too small";
        case GMM_E_HIP: return "HIP runtime error";
        case GMM_E_NOT_PD: return "covariance not positive definite";
        case GMM_E_NONFINITE: return "non-finite result";
    }
    return "unknown status";
}

const char* gmm_version(void) { return "0.1.0"; }

}  // extern "C"
