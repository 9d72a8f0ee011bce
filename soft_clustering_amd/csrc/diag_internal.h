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

// Fused-kernel launch configuration: one workgroup per CU (grid = CUs,
// capped by the partial slots and by the number of 32-point tiles), each
// wave walking its own run of tiles.  Each wave holds a 32-point tile pair
// (fp16 hi / lo, 16 KB for D <= 64, 32 KB for D = 128) in LDS and the split
// panel plus the statistic accumulators in registers: eight waves (two per
// SIMD) while that fits 256 registers per lane, else four.
constexpr int kDiagWgPerCu = 1;
__host__ __device__ constexpr int diag_split_waves(int dp, int kb) {
    return (dp <= 64 && dp * kb <= 64) ? 8 : 4;
}

// Tiles one wave accumulates in fp32 before its run is closed: the E+M pass
// is launched in segments of at most this many tiles per wave, each adding
// its fp32 sums into the workgroups' fp64 partial slots.
constexpr int64_t kDiagSegTiles = 256;

// |y| bound of the split-fp16 operands: y^2 stays below the fp16 maximum
// (65504) with margin; a tile with any larger |y| takes the fp32 route.
constexpr float kSplitLim = 224.0f;


// Threads of the reduction / M-step kernel (one workgroup per component and
// 32-dimension chunk): sixteen waves, so that each wave's strided walk over
// the partial slots is short.
constexpr int kDiagReduceThreads = 1024;

// Dimensions per chunk of the M-step / normaliser sums.
constexpr int kDiagChunkDims = 32;
inline int diag_chunks(const Plan& p) { return (int)((p.d + kDiagChunkDims - 1) / kDiagChunkDims); }

struct DiagWs {
    float *pi, *mu, *var, *panel;
    float *shift, *scale;   // [DP] centre c and power-of-two scale s: y = (x - c) s
                            // (s: written by the fused kernel for its reduction)
    double *part, *part_ll, *stats, *ll;
    int *flags, *retries, *nonfinite_ll;
    int* done;              // workgroups of the running fused kernel that have finished
    double* chunk_part;   // [K][chunks][4]: sum log var, sum (mu-c)^2/var, #bad, #non-finite
};

inline DiagWs diag_ws(const Plan& p, char* ws) {
    DiagWs w;
    w.pi = (float*)(ws + p.off_pi);
    w.mu = (float*)(ws + p.off_mu);
    w.var = (float*)(ws + p.off_cov);
    w.shift = (float*)(ws + p.off_shift);
    w.scale = w.shift + p.dp;
    w.panel = (float*)(ws + p.off_panel);
    w.part = (double*)(ws + p.off_part);
    w.part_ll = (double*)(ws + p.off_part_ll);
    w.stats = (double*)(ws + p.off_stats);
    w.ll = (double*)(ws + p.off_ll);
    w.flags = (int*)(ws + p.off_diag);
    w.retries = w.flags + p.k;
    w.nonfinite_ll = w.flags + 2 * p.k;
    w.done = w.flags + 2 * p.k + 1;
    w.chunk_part = (double*)(ws + p.off_chunk);
    return w;
}

// Number of workgroups (= partial slots) of the fused kernel for this plan.
int diag_grid(const Plan& p);

// Top-m output of the E-step alone (m = 0: none): out_idx / out_gamma [N][m].
struct DiagTopm {
    int m;
    int* idx;
    float* gamma;
};

// Launch the fused split-fp16 kernel (diag_split.hip): EM = statistics
// partials (moments of y = (x - c) s, undone by the reduction); otherwise
// E-step only with optional per-point outputs (LSE, argmax, top-m).  Either
// way the kernel leaves the LL in the workspace and in ll_out (nullable).
hipError_t diag_launch_split(const Plan& p, const DiagWs& w, const void* x, bool em, int grid,
                             double* ll_out, float* lse, int* arg, const DiagTopm& tm,
                             hipStream_t s);

}  // namespace gmm
