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
// Added to LK_SWEEP1 / LK_FUSED_E when the per-point argmax is wanted: the
// comparisons it needs are compiled only into those variants.
constexpr int kLkArg = 8;
// Added to LK_SWEEP1 when the number of slices is even: one workgroup of
// eight waves scores two slices, so each tile is staged once for both.
constexpr int kLkPair = 16;

// Largest m of gmm_assign.
constexpr int kLkMaxTopm = 16;

// fp16 operand range: squares and entries are clamped / scaled below this.
constexpr float kF16Max = 65504.0f;

// A component whose estimated fp16 score rounding error near its own mean
// exceeds this many nats is flagged (bit 4) and scored in the exact centred
// form instead of the panel.  Score errors of e nats shift a responsibility's
// log-odds by up to about e: at one nat a point shared by two components can
// move a sizeable part of its weight, so the bar stays there; typical
// well-conditioned components estimate a few tenths of a nat.
constexpr double kLkIllCondNats = 1.0;

// Tiles one workgroup accumulates in fp32 before its run is closed: the
// statistics passes are launched in segments of at most this many tiles per
// point chunk, and each segment adds its fp32 sums into the workgroup's fp64
// partial slot.
constexpr int64_t kLkSegTiles = 4096;

// Exactly scored components (largek_exact.hip): workgroups of the statistics
// kernel, and the fp64 slot area it writes (at least one slot of every
// listed component; more slots when fewer components are listed).
constexpr int kLkXcSlots = 256;
constexpr size_t kLkXcSlotBytes = (size_t)32 << 20;
inline size_t lk_xc_part_bytes(int64_t k, int64_t ncol) {
    const size_t one = sizeof(double) * (size_t)k * ncol;
    return one > kLkXcSlotBytes ? one : kLkXcSlotBytes;
}
// Slots in use for nx listed components: as many as fit, at most `grid`.
__host__ __device__ inline int lk_xc_slots(int nx, int64_t ncol, int64_t slot_doubles, int grid) {
    if (nx <= 0) return 0;
    int64_t P = slot_doubles / ((int64_t)nx * ncol);
    if (P < 1) P = 1;
    return (int)(P < grid ? P : grid);
}

// Slots for per-workgroup LL partials and range flags (fused kernel and the
// slice-merge kernel), and workgroups of the slice-merge kernel.
constexpr int kLkLLSlots = 1024;
constexpr int kLkMergeWgs = 1024;

// Rows of X sampled for the centre / scale, and workgroups scanning them.
constexpr int kLkScanRows = 4096;
constexpr int kLkScanWgs = 256;   // 16 sample rows per workgroup: the scattered row reads all in flight

struct LkWs {
    float *pi, *mu, *var;        // fp32 parameters theta (var: [K] iso, [K*D] diag)
    float2* dsc;                 // [DP] (c_d, s_d): y' = (x - c_d) * s_d, s_d = 2^-e_d
    float* scan;                 // [scan workgroups][DP][3] sample (sum, min, max)
    uint4* panel;                // fp16 score panel, MFMA A-operand register layout
    float* kmax;                 // [Kpad] largest panel magnitude of each component
    float* prm;                  // [4] panel scale F = 2^f, |y|^2 scale 2^-g, 2^g, unused
    float* c0;                   // [Kpad] base-2 constant of the centred-form score
    float* part_lse;             // [S + 1][N] base-2 LSE of each slice and (row S) of the
                                 // exactly scored components; row 0 then holds the
                                 // merged LSE
    int* part_arg;               // [S + 1][N] argmax within each slice / row
    float* part_max;             // [S + 1][N] largest score within each slice / row
    int *xc_idx, *xc_pos, *xc_n; // exactly scored components: list [K], position of
                                 // each component in it (-1: panel) [K], count
    double* xc_part;             // their statistics slots
    int64_t xc_slot_doubles;
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
    w.c0 = w.prm + 4;
    w.part_lse = (float*)(ws + p.off_lse);
    w.part_arg = (int*)(ws + p.off_arg);
    w.part_max = (float*)(w.part_arg + (size_t)(p.lk_slices + 1) * p.n);
    w.xc_idx = (int*)(ws + p.off_xc);
    w.xc_pos = w.xc_idx + p.k;
    w.xc_n = w.xc_pos + p.k;
    w.xc_part = (double*)(ws + p.off_xcpart);
    w.xc_slot_doubles = (int64_t)(lk_xc_part_bytes(p.k, p.ncols) / sizeof(double));
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
    // exactly scored components: count; one slice: their per-point base-2 LSE,
    // largest score and argmax (row S of part_lse / part_max / part_arg), and
    // where the fused kernels write the merged LSE for their statistics
    const int* xc_n;
    const float *xlse, *xmax;
    const int* xarg;
    float* lse_out;
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
    mode &= kLkArg - 1;
    return ((mode == LK_FUSED_EM || mode == LK_SWEEP2) && cov == GMM_COV_ISO) ? 8 : 4;
}

// Workgroups per CU of the fused kernel: the modes without statistics
// accumulators fit two workgroups (two waves per SIMD, so one wave's MFMAs
// overlap the other's vector work and latencies); the statistics modes need
// up to 512 registers per lane and run one.
__host__ __device__ constexpr int lk_wg_per_cu(int mode) {
    if (mode & kLkPair) return 1;   // eight waves: two per SIMD already
    mode &= kLkArg - 1;
    return (mode == LK_SWEEP1 || mode == LK_FUSED_E) ? 2 : 1;
}

// Slices per workgroup and threads per workgroup of a mode (with its bits).
__host__ __device__ constexpr int lk_slices_per_wg(int mode) { return (mode & kLkPair) ? 2 : 1; }
__host__ __device__ constexpr int lk_threads(int mode, int cov) {
    return 64 * lk_waves(mode, cov) * lk_slices_per_wg(mode);
}

// The variant bits that depend on the plan only (not on the call's outputs).
inline int lk_plan_mode(const Plan& p, int mode) {
    return (mode == LK_SWEEP1 && p.lk_slices % 2 == 0) ? (mode | kLkPair) : mode;
}

// Workgroups of the fused kernel in `mode` (chunks x slices), a function of
// the plan and the device only.
int lk_grid(const Plan& p, int mode);

// Launch the fused kernel in `mode` (largek.hip).
hipError_t lk_launch(const Plan& p, const LkArgs& a, int mode, int grid, hipStream_t s);

// The exactly scored components (largek_exact.hip).
hipError_t lk_xc_build(const Plan& p, const LkWs& w, hipStream_t s);
hipError_t lk_xc_lse(const Plan& p, const LkWs& w, const void* x, hipStream_t s);
hipError_t lk_xc_stats(const Plan& p, const LkWs& w, const void* x, hipStream_t s);
hipError_t lk_xc_topm(const Plan& p, const LkWs& w, const void* x, int m, int* idx, float* score,
                      hipStream_t s);

// Workgroup index of (slice, chunk) in a grid of G = chunks * S workgroups
// (XCD-aware when G is a multiple of 8 * S: the slices of one chunk share
// blockIdx % 8, i.e. one XCD and its L2).
__host__ __device__ inline int lk_wg_of(int slice, int chunk, int G, int S) {
    if (G % (8 * S) == 0) return 8 * ((chunk / 8) * S + slice) + (chunk % 8);
    return chunk * S + slice;
}

}  // namespace gmm
