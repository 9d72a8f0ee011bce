// Internal interface between the diagonal-covariance kernels: workspace
// pointers, the supported (padded D, component-block) shapes and the launch
// configuration of the fused E+M kernel.
#pragma once

#include "common.h"
#include "plan.h"

namespace gmm {

// (DP, KB): D padded to DP in {16, 32, 64, 128}, K padded to 16*KB.
#define GMM_DIAG_SHAPES(X) \
    X(16, 1) X(16, 2) X(16, 3) X(16, 4) X(32, 1) X(32, 2) X(32, 3) X(32, 4) X(64, 1) X(64, 2) X(128, 1)

// Fused-kernel launch configuration: waves per workgroup (each wave walks its
// own run of 16-point groups through a 3-slot LDS ring) and one workgroup per
// CU (grid = CUs, capped by the partial slots and by the number of groups).
// Eight waves (two per SIMD) when the ring fits in LDS (D <= 64: 104 KB),
// four for D = 128 (101 KB).  Measured on the 1e6 x 64 x 16 workload:
// 8 waves x 1 workgroup/CU 108 us, 4 x 2 111 us, 4 x 1 118 us, 2 x 2 182 us.
constexpr int diag_waves(int dp) { return dp <= 64 ? 8 : 4; }
constexpr int kDiagWgPerCu = 1;

// Dimensions per chunk of the M-step / normaliser sums.
constexpr int kDiagChunkDims = 32;
inline int diag_chunks(const Plan& p) { return (int)((p.d + kDiagChunkDims - 1) / kDiagChunkDims); }

struct DiagWs {
    float *pi, *mu, *var, *shift, *panel;
    double *part, *part_ll, *stats, *ll;
    int *flags, *retries, *nonfinite_ll;
    double* chunk_part;   // [K][chunks][4]: sum log var, sum (mu-c)^2/var, #bad, #non-finite
};

inline DiagWs diag_ws(const Plan& p, char* ws) {
    DiagWs w;
    w.pi = (float*)(ws + p.off_pi);
    w.mu = (float*)(ws + p.off_mu);
    w.var = (float*)(ws + p.off_cov);
    w.shift = (float*)(ws + p.off_shift);
    w.panel = (float*)(ws + p.off_panel);
    w.part = (double*)(ws + p.off_part);
    w.part_ll = (double*)(ws + p.off_part_ll);
    w.stats = (double*)(ws + p.off_stats);
    w.ll = (double*)(ws + p.off_ll);
    w.flags = (int*)(ws + p.off_diag);
    w.retries = w.flags + p.k;
    w.nonfinite_ll = w.flags + 2 * p.k;
    w.chunk_part = (double*)(ws + p.off_chunk);
    return w;
}

// Number of workgroups (= partial slots) of the fused kernel for this plan.
int diag_grid(const Plan& p);

// Launch the fused kernel: EM = statistics + LL partials; otherwise E-step
// only with optional per-point outputs.  Defined in diag_fused.hip.
hipError_t diag_launch_fused(const Plan& p, const DiagWs& w, const void* x, bool em, int grid,
                             float* lse, int* arg, hipStream_t s);

}  // namespace gmm
