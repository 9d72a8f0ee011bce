// Internal interface of the large-K family (isotropic or diagonal covariance,
// X stored in bf16 or fp16, fp16 MFMA operands (v_mfma_f32_32x32x16_f16),
// fp32 softmax and statistics): workspace pointers, kernel arguments and
// launch helpers.
#pragma once

#include "common.h"
#include "plan.h"

namespace gmm {

// Points per tile and components per workgroup (slice) of the fused kernel.
constexpr int kLkT = 32;
constexpr int kLkSlice = 256;

// Fused-kernel variants.
enum LkMode : int {
    LK_FUSED_EM = 0,   // K fits one slice: LSE and statistics in one sweep
    LK_SWEEP1 = 1,     // per (slice, point) base-2 LSE (+ argmax) over the slice
    LK_SWEEP2 = 2,     // merge the slices' LSE, statistics of this slice
    LK_FUSED_E = 3,    // K fits one slice: E-step only (LL, per-point outputs)
    LK_TOPM = 4,       // one slice per launch: the m largest responsibilities per
                       // point, merged with those of the slices before it
};

// Largest m of gmm_assign.
constexpr int kLkMaxTopm = 16;

// fp16 operand range: squares and entries are clamped / scaled below this.
constexpr float kF16Max = 65504.0f;

// A component whose estimated score rounding error near its own mean exceeds
// this many nats is reported as ill-conditioned (flag bit 4).
constexpr double kLkIllCondNats = 4.0;

// Tiles one workgroup accumulates in fp32 before its run is closed: the
// statistics passes are launched in segments of at most this many tiles per
// point chunk, and each segment adds its fp32 sums into the workgroup's fp64
// partial slot.
constexpr int64_t kLkSegTiles = 4096;

// Slots for per-workgroup LL partials and range flags (fused kernel and the
// slice-merge kernel), and workgroups of the slice-merge kernel.
constexpr int kLkLLSlots = 1024;
constexpr int kLkMergeWgs = 1024;

// Rows of X sampled for the centre / scale, and workgroups scanning them.
constexpr int kLkScanRows = 4096;
constexpr int kLkScanWgs = 32;

struct LkWs {
    float *pi, *mu, *var;        // fp32 parameters theta (var: [K] iso, [K*D] diag)
    float2* dsc;                 // [DP] (c_d, s_d): y' = (x - c_d) * s_d, s_d = 2^-e_d
    float* scan;                 // [scan workgroups][DP][3] sample (sum, min, max)
    uint4* panel;                // fp16 score panel, MFMA A-operand register layout
    float* kmax;                 // [Kpad] largest panel magnitude of each component
    float* prm;                  // [4] panel scale F = 2^f, |y|^2 scale 2^-g, 2^g, unused
    float* part_lse;             // [S][N] base-2 LSE of each slice; row 0 is then
                                 // overwritten with the merged LSE (two sweeps, and
                                 // top-m assignment at any S)
    int* part_arg;               // [S][N] argmax within each slice (two-sweep only)
    float* part_max;             // [S][N] largest score within each slice
    double *part, *part_ll;      // per-workgroup partials
    int* part_flag;              // per workgroup: X outside the fp16 operand range
    double *stats, *ll;          // reduced statistics (raw moments), LL
    int* flags;                  // [K] bit0 bad params, bit2 empty, bit3 non-finite,
                                 //     bit4 ill-conditioned fp16 score
    int* misc;                   // [0] non-finite LL, [1] X outside the fp16 operand range
};

inline LkWs lk_ws(const Plan& p, char* ws) {
    LkWs w;
    w.pi = (float*)(ws + p.off_pi);
    w.mu = (float*)(ws + p.off_mu);
    w.var = (float*)(ws + p.off_cov);
    w.dsc = (float2*)(ws + p.off_shift);
    w.scan = (float*)(w.dsc + p.dp);
    w.panel = (uint4*)(ws + p.off_panel);
    w.kmax = (float*)(ws + p.off_chunk);
    w.prm = w.kmax + p.lk_kpad;
    const bool two = p.lk_slices > 1;
    w.part_lse = (float*)(ws + p.off_lse);
    w.part_arg = two ? (int*)(ws + p.off_arg) : nullptr;
    w.part_max = two ? (float*)(w.part_arg + (size_t)p.lk_slices * p.n) : nullptr;
    w.part = (double*)(ws + p.off_part);
    w.part_ll = (double*)(ws + p.off_part_ll);
    w.part_flag = (int*)(w.part_ll + kLkLLSlots);
    w.stats = (double*)(ws + p.off_stats);
    w.ll = (double*)(ws + p.off_ll);
    w.flags = (int*)(ws + p.off_diag);
    w.misc = w.flags + 2 * p.k;   // after [K] flags and [K] ridge retries (unused here)
    return w;
}

// Arguments of the fused kernel (one struct, passed by value).
struct LkArgs {
    const void* x;
    int64_t n, ldx;
    int d, k_real, S, vec;
    const uint4* panel;
    int nblk;                    // 32-component blocks in the panel (Kpad / 32)
    const float* prm;            // panel scale and |y|^2 scales (LkWs::prm)
    const float2* dsc;
    float* part_lse;             // sweep 1 output [S][N] (base-2 LSE per slice)
    int* part_arg;               // sweep 1 output [S][N] (nullable: no argmax)
    float* part_max;             // sweep 1 output [S][N] (with part_arg)
    const float* lse_in;         // sweep 2 input [N]: merged base-2 LSE
    double* part;
    double* part_ll;
    int* part_flag;
    float* out_lse;              // E-only: natural-log LSE per point (nullable)
    int* out_arg;                // E-only: argmax per point (nullable)
    // segment: tiles [tlo, thi) split over the point chunks; the first
    // segment writes the partial slots, later ones add to them
    int64_t tlo, thi;
    int seg_first;
    // top-m mode: slice of this launch, m, outputs [N][m] (between slices
    // out_gamma holds base-2 scores; the last slice turns them into
    // responsibilities with lse_in)
    int topm, topm_slice;
    int* out_idx;
    float* out_gamma;
};

// Segments of a statistics pass: tiles split into `nseg` ranges of nearly
// equal length, each at most seg_tiles per chunk.
struct LkSegs {
    int64_t tiles, len;
    int n;
};
inline LkSegs lk_segs(int64_t n_points, int chunks, int64_t seg_tiles) {
    LkSegs s;
    s.tiles = (n_points + kLkT - 1) / kLkT;
    const int64_t per = (int64_t)chunks * (seg_tiles > 0 ? seg_tiles : 1);
    s.n = (int)((s.tiles + per - 1) / per);
    if (s.n < 1) s.n = 1;
    s.len = (s.tiles + s.n - 1) / s.n;
    return s;
}

// Statistic columns per component: diag [s0, s1(D), s2(D)], iso [s0, s1(D), s2].
inline int64_t lk_ncols(int cov, int64_t d) { return cov == GMM_COV_ISO ? 2 + d : 1 + 2 * d; }

// Waves per workgroup of the fused kernel.  The isotropic statistics modes
// run 8 waves of 32 components (one 32-component MFMA block each): at two
// waves per SIMD each wave's panel, accumulators and operands fit 256
// registers and the two waves hide each other's latencies (1e7 x 128 x 256:
// 3.47 -> 2.82 ms).  The diagonal statistics modes keep 4 waves of 64
// components, one per SIMD (at 8 waves the D = 128 variant spills and reads
// the tile twice as often: sweep 2 of 2e8 x 128 x 1024 went 253 -> 272 ms).
// The modes without statistics run 4 waves and two workgroups per CU.
__host__ __device__ constexpr int lk_waves(int mode, int cov) {
    return ((mode == LK_FUSED_EM || mode == LK_SWEEP2) && cov == GMM_COV_ISO) ? 8 : 4;
}

// Workgroups per CU of the fused kernel: the modes without statistics
// accumulators fit two workgroups (two waves per SIMD, so one wave's MFMAs
// overlap the other's vector work and latencies); the statistics modes need
// up to 512 registers per lane and run one.
__host__ __device__ constexpr int lk_wg_per_cu(int mode) {
    return (mode == LK_SWEEP1 || mode == LK_FUSED_E) ? 2 : 1;
}

// Workgroups of the fused kernel in `mode` (chunks x slices), a function of
// the plan and the device only.
int lk_grid(const Plan& p, int mode);

// Launch the fused kernel in `mode` (largek.hip).
hipError_t lk_launch(const Plan& p, const LkArgs& a, int mode, int grid, hipStream_t s);

// Workgroup index of (slice, chunk) in a grid of G = chunks * S workgroups
// (XCD-aware when G is a multiple of 8 * S: the slices of one chunk share
// blockIdx % 8, i.e. one XCD and its L2).
__host__ __device__ inline int lk_wg_of(int slice, int chunk, int G, int S) {
    if (G % (8 * S) == 0) return 8 * ((chunk / 8) * S + slice) + (chunk % 8);
    return chunk * S + slice;
}

}  // namespace gmm
