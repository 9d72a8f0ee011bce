// Internal interface of the full-covariance family: X stored in fp16 (or
// bf16 / fp32), per-component Cholesky factors L stored in fp16, fp32 forward
// solve on the vector unit, fp16 MFMA for the second-moment statistics.
#pragma once

#include "common.h"
#include "plan.h"

namespace gmm {

constexpr int kFullKP = 16;        // components per launch (K <= 16, padded to 16)
constexpr int kFullT = 256;        // points per tile: one per thread
constexpr int kFullLLSlots = 512;  // per-workgroup LL partial slots

// Halves per packed row of the strictly-lower part of L: row i holds
// L[i][0..i-1], padded to a multiple of 8 so that every row starts on a
// 16-byte boundary.
__host__ __device__ constexpr int full_row_halves(int i) { return (i + 7) / 8 * 8; }
__host__ __device__ constexpr int full_row_off(int i) {
    int o = 0;
    for (int r = 0; r < i; ++r) o += full_row_halves(r);
    return o;
}
__host__ __device__ constexpr int full_l_halves(int dp) { return full_row_off(dp); }

// Packed lower triangle of a D x D symmetric matrix, row-major: (i, j <= i).
__host__ __device__ inline int64_t tri_idx(int64_t i, int64_t j) { return i * (i + 1) / 2 + j; }

struct FullWs {
    float *pi, *mu, *cov;      // fp32 parameters theta (cov [K][D][D])
    uint16_t* lpk;             // [KP][full_l_halves(DP)] fp16 strictly-lower L (scaled)
    float* pdiag;              // [KP][DP] 1 / L_ii (of the fp16-rounded, scaled L)
    float* muh;                // [KP][DP] fp16-rounded mean, as fp32 (the solve's centre)
    float* cvec;               // [KP] base-2 constant log2 pi - 1/2 log2 e (D log 2pi + log|C|)
    float* rscale;             // [KP] 2^-e_k: the solve runs on (x - mu) 2^-e_k against L 2^-e_k
    double *part, *part_ll;    // per-workgroup partials [P][KP][ncolp], [P]
    double *colsum;            // [K][ncolp] reduced partials
    double *stats, *ll;        // [K][1 + D + D*D] raw statistics (full matrices), LL
    int* flags;                // [K] flags, [K] ridge retries, misc[0] non-finite LL
};

inline int64_t full_ncolp(int64_t d) { return 1 + d + d * (d + 1) / 2; }

inline FullWs full_ws(const Plan& p, char* ws) {
    FullWs w;
    w.pi = (float*)(ws + p.off_pi);
    w.mu = (float*)(ws + p.off_mu);
    w.cov = (float*)(ws + p.off_cov);
    w.lpk = (uint16_t*)(ws + p.off_panel);
    char* after = ws + p.off_shift;
    w.pdiag = (float*)after;
    w.muh = w.pdiag + kFullKP * p.dp;
    w.cvec = w.muh + kFullKP * p.dp;
    w.rscale = w.cvec + kFullKP;
    w.part = (double*)(ws + p.off_part);
    w.part_ll = (double*)(ws + p.off_part_ll);
    w.colsum = (double*)(ws + p.off_chunk);
    w.stats = (double*)(ws + p.off_stats);
    w.ll = (double*)(ws + p.off_ll);
    w.flags = (int*)(ws + p.off_diag);
    return w;
}

// Launch the fused kernel (full_fused.hip).  em: statistics + LL partials;
// otherwise E-step only with optional per-point outputs.
hipError_t full_launch_fused(const Plan& p, const FullWs& w, const void* x, bool em, int grid,
                             float* lse, int* arg, hipStream_t s);
int full_grid(const Plan& p);

}  // namespace gmm
