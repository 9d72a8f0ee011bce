// Internal interface of the full-covariance family: X stored in fp16, the
// inverse Cholesky factor of every component as a split fp16 panel,
// whitening and second moments on fp16 MFMA, fp32 softmax and accumulation.
#pragma once

#include "common.h"
#include "plan.h"

namespace gmm {

constexpr int kFullKP = 16;        // components per group and launch (padded to 16)
constexpr int kFullMaxK = 256;     // K <= 256: at most 16 groups
constexpr int kFullT = 256;        // points per tile: one per thread
constexpr int kFullLLSlots = 512;  // per-workgroup LL partial slots

// Whitening panel W = (L s)^{-1} (s = 2^-e the component's power-of-two
// scale) as the A operand of v_mfma_f32_32x32x16_f16: output dimensions in
// blocks of 32 (rows), input dimensions in steps of 16 (K); every entry split
// into fp16 hi and lo parts.  Per component: [hi / lo][out block][K step][64
// lanes] 16-byte vectors, lane l holding row l % 32 and K 8 (l / 32) + e.
__host__ __device__ constexpr int full_nob(int dp) { return dp >= 32 ? dp / 32 : 1; }
__host__ __device__ constexpr int full_nks(int dp) { return dp / 16; }
__host__ __device__ constexpr int full_dpo(int dp) { return 32 * full_nob(dp); }
inline size_t full_w_vecs(int dp) { return (size_t)kFullKP * 2 * full_nob(dp) * full_nks(dp) * 64; }

// Packed lower triangle of a D x D symmetric matrix, row-major: (i, j <= i).
__host__ __device__ inline int64_t tri_idx(int64_t i, int64_t j) { return i * (i + 1) / 2 + j; }

// Components are handled in groups of kFullKP (K padded to KPAD = 16 G).
// With one group the fused kernel forms each point's log-sum-exp itself; with
// several, a first pass writes every group's LSE per point, a merge combines
// them, and the statistics pass of each group normalises with the merged LSE
// (the two loops over the components of [LP-GMM] 3.2).
struct FullWs {
    float *pi, *mu, *cov;      // fp32 parameters theta (cov [K][D][D])
    uint4* wpk;                // whitening panels [KPAD] (see full_nob), hi / lo fp16
    float* wbias;              // [KPAD][dpo] W mu (fp32): z 2^e = W x - W mu
    float* muh;                // [KPAD][DP] fp16-rounded mean, as fp32 (centre of the moments)
    float* cvec;               // [KPAD] base-2 constant log2 pi - 1/2 log2 e (D log 2pi + log|C|)
    float* rscale;             // [KPAD] 2^-e_k: |z|^2 = 2^-2e_k |W x - W mu|^2
    float* part;               // per-workgroup partials [G][P][KP][ncolp] (fp32 accumulators)
    double* part_ll;           // [P] (one group) / merge partials (several groups)
    double *colsum;            // [K][ncolp] reduced partials
    double *stats, *ll;        // [K][1 + D + D*D] raw statistics (full matrices), LL
    int* flags;                // [K] flags, [K] ridge retries, misc[0] non-finite LL
    float* glse;               // several groups: [G][N] natural-log LSE per group; row 0
                               // then holds the merged LSE
    int* garg;                 // several groups: [G][N] argmax within each group (global index)
    float* gmax;               // several groups: [G][N] largest base-2 score within each group
    int groups;
    bool lse_pass;             // the LSE comes from a pass of its own and the merge: several
                               // groups, or D > 64 (statistics launches per quad of components)
    int64_t slots;             // partial slots per group
};

inline int64_t full_ncolp(int64_t d) { return 1 + d + d * (d + 1) / 2; }

inline int full_groups(int64_t k) { return (int)((k + kFullKP - 1) / kFullKP); }

// Whether the statistics pass normalises with a merged LSE written beforehand
// (several groups; or D > 64, where a statistics launch covers four components)
inline bool full_lse_pass(int64_t k, int dp) { return full_groups(k) > 1 || dp > 64; }

inline FullWs full_ws(const Plan& p, char* ws) {
    FullWs w;
    const int kpad = kFullKP * full_groups(p.k);
    w.pi = (float*)(ws + p.off_pi);
    w.mu = (float*)(ws + p.off_mu);
    w.cov = (float*)(ws + p.off_cov);
    w.wpk = (uint4*)(ws + p.off_panel);
    char* after = ws + p.off_shift;
    w.wbias = (float*)after;
    w.muh = w.wbias + kpad * full_dpo(p.dp);
    w.cvec = w.muh + kpad * p.dp;
    w.rscale = w.cvec + kpad;
    w.part = (float*)(ws + p.off_part);
    w.part_ll = (double*)(ws + p.off_part_ll);
    w.colsum = (double*)(ws + p.off_chunk);
    w.stats = (double*)(ws + p.off_stats);
    w.ll = (double*)(ws + p.off_ll);
    w.flags = (int*)(ws + p.off_diag);
    w.groups = full_groups(p.k);
    w.slots = p.p_max;
    w.lse_pass = full_lse_pass(p.k, p.dp);
    w.glse = w.lse_pass ? (float*)(ws + p.off_lse) : nullptr;
    w.garg = w.lse_pass ? (int*)(ws + p.off_arg) : nullptr;
    w.gmax = w.lse_pass ? (float*)(w.garg + (size_t)w.groups * p.n) : nullptr;
    return w;
}

// Kernel arguments that vary by group and pass (see full_launch_fused).
struct FullPass {
    int group;               // components 16 group .. 16 group + 15
    int quad;                // D > 64, statistics launches: components 4 quad .. 4 quad + 3
                             // of the group
    const float* lse_in;     // natural-log LSE per point to normalise with (nullable:
                             // the group's own, when it is the only one)
    float* out_lse;          // E-step: natural-log LSE per point (the group's own)
    int* out_arg;            // E-step: argmax per point (global component index)
    float* out_max;          // E-step: largest base-2 score per point (nullable)
    int topm;                // top-m lists (0: none), merged over the groups in order:
    int* out_idx;            //   [N][m] indices;
    float* out_gamma;        //   [N][m] base-2 scores until the last group, which
    int tm_first, tm_last;   //   turns them into responsibilities with lse_in
};

// Launch the fused kernel (full_fused.hip) over tiles [tlo, thi).  em:
// statistics + LL partials (fp32 partials of this segment; the LL slot is
// written by the first segment and added to by later ones); otherwise E-step
// only with optional per-point outputs.
hipError_t full_launch_fused(const Plan& p, const FullWs& w, const void* x, bool em, int grid,
                             const FullPass& ps, int64_t tlo, int64_t thi, int seg_first,
                             hipStream_t s);
int full_grid(const Plan& p);

// Tiles (of kFullT points) one workgroup accumulates in fp32 before its run
// is closed: the E+M pass runs in segments of at most this many tiles per
// workgroup, and the fp32 partials of each segment are added into fp64
// column sums before the next one.
constexpr int64_t kFullSegTiles = 64;

struct FullSegs {
    int64_t tiles, len;
    int n;
};
inline FullSegs full_segs(const Plan& p, int grid) {
    FullSegs s;
    s.tiles = (p.n + kFullT - 1) / kFullT;
    const int64_t per = (int64_t)grid * (p.seg_tiles > 0 ? p.seg_tiles : kFullSegTiles);
    s.n = (int)((s.tiles + per - 1) / per);
    if (s.n < 1) s.n = 1;
    s.len = (s.tiles + s.n - 1) / s.n;
    return s;
}

}  // namespace gmm
