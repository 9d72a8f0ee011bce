// Host-side plan: validated descriptor, kernel family and workspace layout.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "gmm.h"

namespace gmm {

enum Path : int {
    PATH_DIAG_F32 = 0,   // diagonal, K <= 64: fp32-accurate split-fp16 MFMA scores and statistics
    PATH_LARGEK = 1,     // isotropic / diagonal, X in bf16 or fp16, fp16 MFMA, K <= 4096
    PATH_FULL = 2,       // full covariance, X in fp16, fp16 MFMA whitening and moments, K <= 256, D <= 128
};

struct Plan {
    // descriptor
    int64_t n, d, k, ldx;
    int cov, xdt;
    float var_floor, ridge_rel;
    // kernel choice
    int path;
    int dp;          // D padded to the kernel's dimension tile
    int kb;          // number of 16-component blocks
    int vec;         // 1: 16-byte vector loads of X are legal
    int p_max;       // partial slots reserved in the workspace
    // workspace layout (byte offsets)
    size_t off_pi, off_mu, off_cov;   // fp32 copy of the prepared parameters
    size_t off_shift;                 // per-dimension centre of X
    size_t off_panel;                 // score panel (MFMA register layout)
    size_t off_part, off_part_ll;     // per-workgroup partial statistics
    size_t off_stats, off_ll;         // reduced statistics and LL
    size_t off_diag;                  // status flags, counters
    size_t off_chunk;                 // per-(component, dimension chunk) sums;
                                      // large K: per-component score constants
    size_t off_lse, off_arg;          // large K, two sweeps: per-(slice, point) LSE,
                                      // argmax and maximum
    size_t off_ctl;                   // gmm_fit control block and the start's indices
    size_t off_xc, off_xcpart;        // large K: exactly scored components (list, slots)
    size_t total;
    int64_t ncols;                    // statistic columns per component
    int lk_slices;                    // large K: 256-component slices
    int lk_kpad;                      // large K: K padded to whole slices
    int64_t seg_tiles;                // statistics passes: tiles per workgroup (or wave)
                                      // and launch segment, 0 = the family's default
};

gmm_status make_plan(const gmm_desc* desc, Plan* plan);

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Bytes of the gmm_fit control block (fit.hip).
size_t fit_ctl_bytes(const Plan& p);

// Entry points of the diagonal family (diag_params.hip, diag_split.hip).
gmm_status diag_prepare(const Plan& p, char* ws, const float* pi, const float* mu,
                        const float* var, hipStream_t s);
gmm_status diag_em_step(const Plan& p, char* ws, const void* x, double* ll_out, hipStream_t s);
gmm_status diag_finalize(const Plan& p, char* ws, float* pi, float* mu, float* var,
                         hipStream_t s);
gmm_status diag_loglik(const Plan& p, char* ws, const void* x, double* ll_out, float* lse,
                       int32_t* argmax, hipStream_t s);
gmm_status diag_assign(const Plan& p, char* ws, const void* x, int m, int32_t* idx, float* gamma,
                       double* ll_out, hipStream_t s);
int device_cu_count();

// Entry points of the large-K family (largek_params.hip, largek.hip).
gmm_status lk_prepare(const Plan& p, char* ws, const float* pi, const float* mu,
                      const float* var, hipStream_t s);
gmm_status lk_em_step(const Plan& p, char* ws, const void* x, double* ll_out, hipStream_t s);
gmm_status lk_finalize(const Plan& p, char* ws, float* pi, float* mu, float* var,
                       hipStream_t s);
gmm_status lk_loglik(const Plan& p, char* ws, const void* x, double* ll_out, float* lse,
                     int32_t* argmax, hipStream_t s);
gmm_status lk_assign(const Plan& p, char* ws, const void* x, int m, int32_t* idx, float* gamma,
                     double* ll_out, hipStream_t s);

// Entry points of the full-covariance family (full_params.hip, full_fused.hip).
gmm_status full_prepare(const Plan& p, char* ws, const float* pi, const float* mu,
                        const float* cov, hipStream_t s);
gmm_status full_em_step(const Plan& p, char* ws, const void* x, double* ll_out, hipStream_t s);
gmm_status full_finalize(const Plan& p, char* ws, float* pi, float* mu, float* cov,
                         hipStream_t s);
gmm_status full_loglik(const Plan& p, char* ws, const void* x, double* ll_out, float* lse,
                       int32_t* argmax, hipStream_t s);
gmm_status full_assign(const Plan& p, char* ws, const void* x, int m, int32_t* idx, float* gamma,
                       double* ll_out, hipStream_t s);

}  // namespace gmm
