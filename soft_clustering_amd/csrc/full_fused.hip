// Full-covariance Gaussian mixture, X stored in fp16: fused E-step + M-step
// statistics, one pass over X, no N x K matrix in memory.
//
// Density ([LP-GMM] 1.2, route 2): d^2 = |z|^2 with L z = x - mu.  The
// triangular solve is taken as a product with the inverse factor: z 2^e =
// W x - W mu, W = (L 2^-e)^{-1} formed in fp64 by the preparation kernel and
// stored as fp16 hi + lo parts, so each 32 x 32 block of W x is two
// v_mfma_f32_32x32x16_f16 per K step against the exact fp16 X, accumulated in
// fp32; the bias, |z|^2, exp, log and every normaliser stay fp32 ([LP-GMM]
// 1.3 first boundary); log|C| = 2 sum log L_ii.
// Statistics ([Flash-GMM] Method, s0 / s1 / sum gamma x x^T on chip): s1 =
// gamma^T X and the centred second moment sum_n gamma_nk (x_n - mu_k)
// (x_n - mu_k)^T (lower-triangle 16 x 16 blocks) on fp16 MFMA
// (v_mfma_f32_16x16x32_f16) with fp32 accumulation; the M-step turns them into
// raw moments and the new covariance in fp64.
//
// Work split (k_full_fused, any D): a workgroup of 256 threads takes 256-point
// tiles.  At D = 64 with aligned X, k_full_pipe below splits the same work
// between whitening waves and moment waves instead.  Each thread
// loads one point into the row-major LDS tile (the moments read it
// transposed, with ds_read_b64_tr_b16).
// Phase 1: wave w whitens the tile against components 4w..4w+3 (the
// component's panel in registers, the next component's panel loading behind
// it), writing the base-2 scores to LDS.  Then each thread forms the
// log-sum-exp and the responsibilities of its point.  Phase 2 (E+M only):
// wave w accumulates the second moments of components 4w..4w+3 and the first
// moments of dimension block w over the tile.

#include <type_traits>

#include "full_internal.h"

namespace gmm {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

constexpr int KP = kFullKP;
constexpr int T = kFullT;
constexpr float kLn2f = 0.69314718055994530942f;
constexpr float kHalfLog2e = 0.72134752044448170368f;   // log2(e) / 2

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

// ds_read_b64_tr_b16: in each group of 16 lanes, lane i' reads 4 halves of
// row (i' / 4) at column 4 (i' % 4) (addresses as given); lane i receives
// column i of the 4 rows.
__device__ __forceinline__ uint2 tr16(const uint16_t* p) {
    const short4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)((lds_u16*)p));
    return __builtin_bit_cast(uint2, v);
}

template <int DP>
struct FullShape {
    static constexpr int kNB = DP / 16;                  // 16-dim blocks
    static constexpr int kNBlk = kNB * (kNB + 1) / 2;    // lower-triangle 16 x 16 blocks
    static constexpr int kGS = T + 4;                    // floats per row of the score tile
    static constexpr int kXR = DP + 8;                   // halves per row of the row-major tile
    static constexpr int kNOB = full_nob(DP), kNKS = full_nks(DP), kDPO = full_dpo(DP);
    static constexpr int kNV = 2 * kNOB * kNKS;          // panel vectors per lane and component
};

__device__ __forceinline__ int blk_index(int ab, int bb) { return ab * (ab + 1) / 2 + bb; }

static_assert(KP == 16, "four components per wave, four waves");

// VEC: d % 8 == 0 and 16-byte aligned rows (whole-vector loads); otherwise
// per-element loads.  A template parameter, so that each kernel holds one path.
constexpr int kMaxTopm = 16;
constexpr float kLog2ef = 1.44269504088896340736f;

// Top-m list of point p over this group's KP base-2 scores merged with the
// running list of the groups before it (ps.out_idx / ps.out_gamma, which hold
// base-2 scores until the last group).  Better = larger score, or equal with a
// lower component index (the running entries, from earlier groups, are
// checked first); components scoring -inf (zero weight, padding) are never
// listed: index -1 and 0 past the live ones.  The last group writes the
// responsibilities exp2(score - lse2).
__device__ __forceinline__ void write_topm(const float (&sv)[KP], float lse2, const FullPass& ps,
                                           int64_t p) {
    const int m = ps.topm, k0 = KP * ps.group;
    float rv[kMaxTopm];
    int ri[kMaxTopm];
#pragma unroll
    for (int r = 0; r < kMaxTopm; ++r) {
        const bool ok = !ps.tm_first && r < m;
        ri[r] = ok ? ps.out_idx[p * m + r] : -1;
        rv[r] = (ok && ri[r] >= 0) ? ps.out_gamma[p * m + r] : -INFINITY;
    }
    uint32_t taken = 0;   // bits 0..15: this group's components; 16..31: running entries
#pragma unroll
    for (int i = 0; i < kMaxTopm; ++i) {
        if (i >= m) break;
        float bv = -INFINITY;
        int bk = -1, bs = -1;
#pragma unroll
        for (int r = 0; r < kMaxTopm; ++r)
            if (!((taken >> (16 + r)) & 1u) && ri[r] >= 0 && rv[r] > bv) {
                bv = rv[r];
                bk = ri[r];
                bs = 16 + r;
            }
#pragma unroll
        for (int k = 0; k < KP; ++k)
            if (!((taken >> k) & 1u) && sv[k] > bv) {
                bv = sv[k];
                bk = k0 + k;
                bs = k;
            }
        if (bs >= 0) taken |= 1u << bs;
        ps.out_idx[p * m + i] = bk;
        ps.out_gamma[p * m + i] = bk < 0 ? 0.0f : (ps.tm_last ? fast_exp2(bv - lse2) : bv);
    }
}

template <int DP, bool EM, bool VEC>
__global__ __launch_bounds__(256, 1) void k_full_fused(
    const _Float16* __restrict__ x, int64_t n, int d, int64_t ldx, int k_real,
    const uint4* __restrict__ wpk, const float* __restrict__ wbias, const float* __restrict__ muh,
    const float* __restrict__ cvec, const float* __restrict__ rscale, float* __restrict__ part,
    double* __restrict__ part_ll, const FullPass ps, int64_t tlo, int64_t thi, int seg_first) {
    using Sh = FullShape<DP>;
    constexpr int NB = Sh::kNB, NBLK = Sh::kNBlk;
    constexpr int NOB = Sh::kNOB, NKS = Sh::kNKS, DPO = Sh::kDPO, NV = Sh::kNV;
    __shared__ __attribute__((aligned(16))) uint32_t nm_s[KP][DP];   // (-mu, -mu) as fp16 pairs
    __shared__ __attribute__((aligned(16))) float wb_s[KP][DPO];     // -W mu
    __shared__ float cv_s[KP], hq_s[KP];
    __shared__ __attribute__((aligned(16))) float g_s[KP][Sh::kGS];  // scores, then gamma
    __shared__ __attribute__((aligned(16))) uint16_t xr_s[T][Sh::kXR];   // the tile, row-major
    __shared__ double red[256];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, j = lane & 15;

    // ---- stage the prepared parameters of all components
    for (int i = tid; i < KP * DP; i += 256) {
        const uint32_t h = __builtin_bit_cast(uint16_t, (_Float16)(-muh[i]));
        nm_s[i / DP][i % DP] = h | (h << 16);
    }
    for (int i = tid; i < KP * DPO; i += 256) wb_s[i / DPO][i % DPO] = -wbias[i];
    if (tid < KP) {
        const float rs = rscale[tid];
        cv_s[tid] = cvec[tid];
        hq_s[tid] = kHalfLog2e * rs * rs;   // |z|^2 = 2^-2e |W x - W mu|^2
    }

    const int G = gridDim.x;
    const int64_t tiles = thi - tlo;   // this segment's tiles
    const int64_t tb = tiles / G, tr = tiles % G;
    const int b = blockIdx.x;
    const int64_t t0 = tlo + b * tb + (b < tr ? b : tr);
    const int64_t t1 = t0 + tb + (b < tr ? 1 : 0);

    float s0acc[KP];
#pragma unroll
    for (int k = 0; k < KP; ++k) s0acc[k] = 0.0f;
    f32x4 acc2[EM ? 4 : 1][EM ? NBLK : 1];
    f32x4 acc1 = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (EM) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int q = 0; q < NBLK; ++q) acc2[kk][q] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    double ll = 0.0;

    // One point of tile t (fp16), zero outside [0, N) x [0, D).  Every load is
    // issued unconditionally from an in-bounds address, so the loads of a tile
    // are all in flight together; on the vector path the mask is applied when
    // the tile is stored (`finish`), so that the wait for the loads comes there
    // and not right after them.
    auto load_point = [&](int64_t t, uint4 (&xv)[DP / 8]) __attribute__((always_inline)) {
        const int64_t p = t * T + tid;
        const bool valid = p < n;
        const _Float16* row = x + (valid ? p : 0) * ldx;
        if constexpr (VEC) {
            const int cmax = d / 8;
#pragma unroll
            for (int c = 0; c < DP / 8; ++c)
                xv[c] = *reinterpret_cast<const uint4*>(row + 8 * (c < cmax ? c : 0));
        } else {
            const uint16_t* rb = reinterpret_cast<const uint16_t*>(row);
#pragma unroll
            for (int c = 0; c < DP / 8; ++c) {
                uint32_t wv[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int i0 = 8 * c + 2 * q;
                    const uint32_t lo = rb[i0 < d ? i0 : 0], hi = rb[i0 + 1 < d ? i0 + 1 : 0];
                    wv[q] = (valid && i0 < d ? lo : 0u) | ((valid && i0 + 1 < d ? hi : 0u) << 16);
                }
                xv[c] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
            }
        }
    };
    // The panel of component k (this lane's NV vectors).
    auto load_panel = [&](int k, half8 (&wp)[NV]) __attribute__((always_inline)) {
#pragma unroll
        for (int v = 0; v < NV; ++v)
            wp[v] = __builtin_bit_cast(half8, wpk[((int64_t)k * NV + v) * 64 + lane]);
    };

    auto finish = [&](int64_t t, int c, uint4 v) __attribute__((always_inline)) {
        if constexpr (VEC) {
            const uint32_t m = (t * T + tid < n && c < d / 8) ? ~0u : 0u;
            return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
        } else {
            return v;
        }
    };

    uint4 xv[DP / 8];
    half8 wp[NV];
    if (t0 < t1) {
        load_point(t0, xv);
        load_panel(4 * w, wp);
    }
    for (int64_t t = t0; t < t1; ++t) {
        const int64_t p = t * T + tid;
        const bool valid = p < n;
        __syncthreads();   // the previous tile is done with xr_s / g_s
#pragma unroll
        for (int c = 0; c < DP / 8; ++c) *reinterpret_cast<uint4*>(&xr_s[tid][8 * c]) = finish(t, c, xv[c]);
        __syncthreads();
        if (t + 1 < t1) load_point(t + 1, xv);   // the next tile, behind this one's work

        // ---- phase 1: W x for the components of this wave, 32 points at a time:
        // A = panel (out dimensions x inputs), B = tile rows (inputs x points);
        // lane l holds point l % 32, out dimensions 32 ob + 8 (r / 4) + 4 (l / 32) + r % 4
#pragma unroll 1
        for (int kk = 0; kk < KP / 4; ++kk) {
            const int k = 4 * w + kk;
            half8 wc[NV];
#pragma unroll
            for (int v = 0; v < NV; ++v) wc[v] = wp[v];
            if (kk + 1 < KP / 4) load_panel(k + 1, wp);   // the next component's panel
            else if (t + 1 < t1) load_panel(4 * w, wp);  // the first one of the next tile
            f32x16 nb[NOB];   // -W mu: the accumulators start from it, so they end at W (x - mu)
#pragma unroll
            for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    nb[ob][r] = wb_s[k][32 * ob + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)];
            const float cvk = cv_s[k], hqk = hq_s[k];
#pragma unroll 2
            for (int st = 0; st < T / 32; ++st) {
                f32x16 acc[NOB];
#pragma unroll
                for (int ob = 0; ob < NOB; ++ob) acc[ob] = nb[ob];
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const half8 xb = __builtin_bit_cast(
                        half8, *reinterpret_cast<const uint4*>(&xr_s[32 * st + (lane & 31)][16 * ks + 8 * (lane >> 5)]));
#pragma unroll
                    for (int ob = 0; ob < NOB; ++ob) {
                        if (ks > 2 * ob + 1) continue;   // above the diagonal: W is lower triangular
                        acc[ob] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wc[ob * NKS + ks], xb, acc[ob], 0, 0, 0);
                        acc[ob] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wc[(NOB + ob) * NKS + ks], xb, acc[ob], 0, 0, 0);
                    }
                }
                float q0 = 0.0f, q1 = 0.0f;
#pragma unroll
                for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
                    for (int r = 0; r < 16; r += 2) {
                        q0 = fmaf(acc[ob][r], acc[ob][r], q0);
                        q1 = fmaf(acc[ob][r + 1], acc[ob][r + 1], q1);
                    }
                float q = q0 + q1;
                q = halves_sum(q);
                if (lane < 32) g_s[k][32 * st + lane] = cvk - hqk * q;
            }
        }
        __syncthreads();

        // ---- base-2 log-sum-exp, responsibilities (thread-local)
        {
            float sv[KP];
            float M = -INFINITY;
#pragma unroll
            for (int k = 0; k < KP; ++k) {
                sv[k] = g_s[k][tid];
                M = fmaxf(M, sv[k]);
            }
            const float Ms = M == -INFINITY ? 0.0f : M;
            float Z = 0.0f;
#pragma unroll
            for (int k = 0; k < KP; ++k) Z += fast_exp2(sv[k] - Ms);
            const float own = Ms + fast_log2(Z);
            // several groups: normalise with the merged LSE of all of them
            const float lse2 = ps.lse_in != nullptr ? (valid ? ps.lse_in[p] * kLog2ef : 0.0f) : own;
            if (valid) ll += (double)own;
            if constexpr (EM) {
                const float lsafe = lse2 == -INFINITY ? INFINITY : lse2;   // no live component
#pragma unroll
                for (int k = 0; k < KP; ++k) {
                    const float gk = valid ? fast_exp2(sv[k] - lsafe) : 0.0f;
                    s0acc[k] += gk;
                    g_s[k][tid] = gk;
                }
            } else if (valid) {
                if (ps.out_lse) ps.out_lse[p] = lse2 * kLn2f;
                if (ps.out_arg) {
                    int a = 0;
#pragma unroll
                    for (int k = KP - 1; k >= 0; --k)
                        if (sv[k] == M) a = k;
                    ps.out_arg[p] = KP * ps.group + a;
                }
                if (ps.out_max) ps.out_max[p] = M;
                if (ps.topm > 0) write_topm(sv, lse2, ps, p);
            }
        }

        if constexpr (EM) {
            __syncthreads();
            // ---- phase 2: second moments of components 4w..4w+3, first moments of dims block w
#pragma unroll 1
            for (int ks = 0; ks < T / 32; ++ks) {
                const int pc = 32 * ks + 8 * g;   // this lane's 8 points of the K-step
                // x of points pc..pc+7, dimension 16 bb + j: two transposed reads of the tile
                uint4 xb[NB];
#pragma unroll
                for (int bb = 0; bb < NB; ++bb) {
                    const uint16_t* src = &xr_s[32 * ks + 8 * g + (j >> 2)][16 * bb + 4 * (j & 3)];
                    const uint2 lo = tr16(src), hi = tr16(src + 4 * Sh::kXR);
                    xb[bb] = make_uint4(lo.x, lo.y, hi.x, hi.y);
                }
                if (w < NB) {   // s1 += gamma^T x over all components, dims 16w..16w+15
                    const float4 g0 = *reinterpret_cast<const float4*>(&g_s[j][pc]);
                    const float4 g1 = *reinterpret_cast<const float4*>(&g_s[j][pc + 4]);
                    const half8 ga = {(_Float16)g0.x, (_Float16)g0.y, (_Float16)g0.z, (_Float16)g0.w,
                                      (_Float16)g1.x, (_Float16)g1.y, (_Float16)g1.z, (_Float16)g1.w};
                    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ga, __builtin_bit_cast(half8, xb[w]), acc1, 0, 0, 0);
                }
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int k = 4 * w + kk;
                    const float4 g0 = *reinterpret_cast<const float4*>(&g_s[k][pc]);
                    const float4 g1 = *reinterpret_cast<const float4*>(&g_s[k][pc + 4]);
                    const half8 gh = {(_Float16)g0.x, (_Float16)g0.y, (_Float16)g0.z, (_Float16)g0.w,
                                      (_Float16)g1.x, (_Float16)g1.y, (_Float16)g1.z, (_Float16)g1.w};
                    half8 yc[NB], ya[NB];
#pragma unroll
                    for (int bb = 0; bb < NB; ++bb) {
                        const half2v nm = __builtin_bit_cast(half2v, nm_s[k][16 * bb + j]);
                        const half8 x8 = __builtin_bit_cast(half8, xb[bb]);
                        // x + (-mu): an add of the splatted pair stays on v_pk_add_f16
                        yc[bb] = x8 + __builtin_shufflevector(nm, nm, 0, 1, 0, 1, 0, 1, 0, 1);
                        ya[bb] = yc[bb] * gh;   // gamma (x - mu_k)
                    }
#pragma unroll
                    for (int ab = 0; ab < NB; ++ab)
#pragma unroll
                        for (int bb = 0; bb <= ab; ++bb)
                            acc2[kk][blk_index(ab, bb)] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                ya[ab], yc[bb], acc2[kk][blk_index(ab, bb)], 0, 0, 0);
                }
            }
        }
    }

    // ---- epilogue: per-workgroup partials [KP][1 + D + D(D+1)/2], one writer each
    __syncthreads();
    if constexpr (EM) {
        const int ncolp = 1 + d + d * (d + 1) / 2;
        float* dst = part + (int64_t)b * KP * ncolp;   // fp32: the accumulators' own precision
#pragma unroll
        for (int k = 0; k < KP; ++k) g_s[k][tid] = s0acc[k];
        __syncthreads();
        if (tid < KP) {
            double s = 0.0;
            for (int i = 0; i < T; ++i) s += (double)g_s[tid][i];
            dst[(int64_t)tid * ncolp] = (float)s;
        }
        if (w < NB) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int k = 4 * g + r, dd = 16 * w + j;
                if (dd < d) dst[(int64_t)k * ncolp + 1 + dd] = acc1[r];
            }
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int k = 4 * w + kk;
#pragma unroll
            for (int ab = 0; ab < NB; ++ab)
#pragma unroll
                for (int bb = 0; bb <= ab; ++bb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = 16 * ab + 4 * g + r, col = 16 * bb + j;
                        if (row >= col && row < d)
                            dst[(int64_t)k * ncolp + 1 + d + tri_idx(row, col)] =
                                acc2[kk][blk_index(ab, bb)][r];
                    }
        }
    }
    red[tid] = ll;
    __syncthreads();
    for (int s2 = 128; s2 > 0; s2 >>= 1) {
        if (tid < s2) red[tid] += red[tid + s2];
        __syncthreads();
    }
    if (tid == 0 && part_ll != nullptr) part_ll[b] = seg_first ? red[0] * kLn2 : part_ll[b] + red[0] * kLn2;
}

// ---------------------------------------------------------------------------
// D = 64: a two-stage pipeline over 256-point tiles in one workgroup of 12
// waves (three per SIMD).  Waves 0..3 whiten tile i (components 4w..4w+3, as
// above) and stage tile i + 1 into LDS; waves 4..11 take tile i - 1: every one
// forms the base-2 log-sum-exp of all 256 points from the 16 scores, keeps the
// responsibilities of its two components (2v, 2v + 1) in a private LDS row, and
// accumulates their first and second moments.  One barrier per tile; three tile
// buffers (the whitened tile, the tile of the moments, the tile being staged)
// and two score buffers.  A SIMD thus holds one whitening wave and two moment
// waves, whose vector and matrix work overlap.
namespace pipe {
constexpr int kWaves = 12;
constexpr int kThreads = 64 * kWaves;
constexpr int DP = 64, NB = 4, NBLK = 10, NOB = 2, NKS = 4, DPO = 64, NV = 16;
constexpr int kGS = T + 4;
// 16-byte unit u of tile row r sits at unit u ^ ((r >> 1) & 7): 16 consecutive
// rows read at one logical unit fall on 16 distinct (bank half, unit) pairs
__device__ __forceinline__ int xoff(int r, int u) { return r * DP + 8 * (u ^ ((r >> 1) & 7)); }
}  // namespace pipe

template <bool EM, bool EXT>   // EXT: normalise with the merged LSE of several groups
__global__ __launch_bounds__(pipe::kThreads, 1) void k_full_pipe(
    const _Float16* __restrict__ x, int64_t n, int d, int64_t ldx, int k_real,
    const uint4* __restrict__ wpk, const float* __restrict__ wbias, const float* __restrict__ muh,
    const float* __restrict__ cvec, const float* __restrict__ rscale, float* __restrict__ part,
    double* __restrict__ part_ll, const FullPass ps, int64_t tlo, int64_t thi, int seg_first) {
    using namespace pipe;
    __shared__ __attribute__((aligned(16))) uint32_t nm_s[KP][DP];     // (-mu, -mu) fp16 pairs
    __shared__ __attribute__((aligned(16))) float wb_s[KP][NOB][2][16];  // -W mu, accumulator layout
    __shared__ float cv_s[KP], hq_s[KP];
    __shared__ __attribute__((aligned(16))) float g_s[2][KP][kGS];     // scores of two tiles
    __shared__ __attribute__((aligned(16))) uint16_t xr_s[3][T * DP];  // three tiles, swizzled
    __shared__ __attribute__((aligned(16))) uint16_t gp_s[EM ? 8 : 1][2][T + 8];   // fp16 gamma, per moment wave

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, j = lane & 15;
    const bool p1 = w < 4;
    const int v = w - 4;   // moment wave index (0..7)

    for (int i = tid; i < KP * DP; i += kThreads) {
        const uint32_t h = __builtin_bit_cast(uint16_t, (_Float16)(-muh[i]));
        nm_s[i / DP][i % DP] = h | (h << 16);
    }
    for (int i = tid; i < KP * NOB * 32; i += kThreads) {
        const int k = i / (NOB * 32), ob = (i / 32) % NOB, hh = (i / 16) % 2, r = i % 16;
        wb_s[k][ob][hh][r] = -wbias[k * DPO + 32 * ob + 8 * (r >> 2) + 4 * hh + (r & 3)];
    }
    if (tid < KP) {
        const float rs = rscale[tid];
        cv_s[tid] = cvec[tid];
        hq_s[tid] = kHalfLog2e * rs * rs;
    }

    const int G = gridDim.x;
    const int64_t tiles = thi - tlo;   // this segment's tiles
    const int64_t tb = tiles / G, tr = tiles % G;
    const int b = blockIdx.x;
    const int64_t t0 = tlo + b * tb + (b < tr ? b : tr);
    const int nt = (int)(tb + (b < tr ? 1 : 0));

    // the whitening stage's point loads: thread tid < 256 holds point tid of a
    // tile, loaded raw from an in-bounds address and masked when stored (so
    // that the wait for the loads comes at the store, a tile later)
    uint4 xv[8];
    auto load_point = [&](int64_t t) __attribute__((always_inline)) {
        const int64_t p = t * T + tid;
        const _Float16* row = x + (p < n ? p : 0) * ldx;
        const int cmax = d / 8;
#pragma unroll
        for (int c = 0; c < 8; ++c) xv[c] = *reinterpret_cast<const uint4*>(row + 8 * (c < cmax ? c : 0));
    };
    auto store_point = [&](int buf, int64_t t) __attribute__((always_inline)) {
        const bool valid = t * T + tid < n;
        const int cmax = d / 8;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const uint32_t m = (valid && c < cmax) ? ~0u : 0u;
            *reinterpret_cast<uint4*>(&xr_s[buf][xoff(tid, c)]) =
                make_uint4(xv[c].x & m, xv[c].y & m, xv[c].z & m, xv[c].w & m);
        }
    };

    if (p1) {
        // ---- whitening stage: stages tile it + 1, loads tile it + 2, whitens tile it
        if (nt > 0) {
            load_point(t0);
            store_point(0, t0);
            if (nt > 1) load_point(t0 + 1);
        }
        __syncthreads();
        for (int it = 0; it <= nt; ++it) {
            if (it < nt) {
                if (it + 1 < nt) store_point((it + 1) % 3, t0 + it + 1);
                if (it + 2 < nt) load_point(t0 + it + 2);
                const uint16_t* xt = xr_s[it % 3];
                float(*gs)[kGS] = g_s[it & 1];
#pragma unroll 1
                for (int kk = 0; kk < KP / 4; ++kk) {
                    const int k = 4 * w + kk;
                    half8 wp[NV];
#pragma unroll
                    for (int vv = 0; vv < NV; ++vv) {
                        const int ks = vv % NKS, ob = (vv / NKS) % NOB;
                        if (ks > 2 * ob + 1) continue;   // above the diagonal
                        wp[vv] = __builtin_bit_cast(half8, wpk[((int64_t)k * NV + vv) * 64 + lane]);
                    }
                    const float cvk = cv_s[k], hqk = hq_s[k];
                    // Point blocks st = 0 .. 7 of 32 points, software-pipelined.  Per
                    // block the 4 MFMAs of output block 0 (inputs 0..31) come first,
                    // then the 8 of output block 1; the squares of output block 0
                    // are summed between the MFMAs of output block 1 and those of
                    // output block 1 between the first 4 MFMAs of the next point
                    // block, so the matrix core is not idle while the wave forms
                    // |z|^2.  Each group of FMAs is pinned to its MFMA step: its
                    // operands pass through an empty asm statement there (the
                    // compiler would otherwise place them all after the MFMAs) and
                    // the step ends in a scheduling barrier.
                    f32x16 a0, a1, p1;   // output blocks 0 and 1 of this point block, 1 of the last
                    float q[2][4];       // partial |z|^2 of the last / this point block
                    auto sq = [&](const f32x16& acc, float (&qq)[4], int r0, int r1) __attribute__((always_inline)) {
#pragma unroll
                        for (int r = r0; r < r1; ++r) {
                            float e = acc[r];
                            __asm__ volatile("" : "+v"(e));
                            qq[r % 4] = fmaf(e, e, qq[r % 4]);
                        }
                    };
                    auto finish = [&](float (&qq)[4], int st) __attribute__((always_inline)) {
                        float t = (qq[0] + qq[1]) + (qq[2] + qq[3]);
                        {   // lanes l < 32 add lane l + 32's half (a cross-half swap, no LDS trip)
                            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t),
                                                                             false, false);
                            t += __uint_as_float(sw[1]);
                        }
                        if (lane < 32) gs[k][32 * st + lane] = cvk - hqk * t;
                    };
#pragma unroll
                    for (int st = 0; st <= T / 32; ++st) {
                        float (&qc)[4] = q[st & 1];
                        float (&qp)[4] = q[(st & 1) ^ 1];
                        if (st == T / 32) {   // drain: output block 1 of the last point block
                            sq(p1, qp, 0, 16);
                            finish(qp, st - 1);
                            break;
                        }
                        qc[0] = qc[1] = qc[2] = qc[3] = 0.0f;
                        __asm__ volatile("" ::: "memory");   // -W mu re-read per block
                        a0 = *reinterpret_cast<const f32x16*>(&wb_s[k][0][lane >> 5][0]);
                        a1 = *reinterpret_cast<const f32x16*>(&wb_s[k][1][lane >> 5][0]);
                        const int row = 32 * st + (lane & 31);
                        half8 xb[NKS];
#pragma unroll
                        for (int ks = 0; ks < NKS; ++ks)
                            xb[ks] = __builtin_bit_cast(
                                half8, *reinterpret_cast<const uint4*>(&xt[xoff(row, 2 * ks + (lane >> 5))]));
                        // output block 0: inputs 0..31 (2 steps, hi and lo); squares of the
                        // last point block's output block 1, four per MFMA
#pragma unroll
                        for (int m = 0; m < 4; ++m) {
                            const int ks = m >> 1, hl = m & 1;
                            a0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(wp[(hl * NOB + 0) * NKS + ks], xb[ks], a0, 0, 0, 0);
                            if (st > 0) sq(p1, qp, 4 * m, 4 * m + 4);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                        if (st > 0) finish(qp, st - 1);
                        // output block 1: inputs 0..63 (4 steps, hi and lo); squares of
                        // output block 0 once its chain has completed (from the third MFMA)
#pragma unroll
                        for (int m = 0; m < 8; ++m) {
                            const int ks = m >> 1, hl = m & 1;
                            a1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(wp[(hl * NOB + 1) * NKS + ks], xb[ks], a1, 0, 0, 0);
                            if (m >= 2) sq(a0, qc, (16 * (m - 2)) / 6, (16 * (m - 1)) / 6);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                        p1 = a1;
                    }
                }
            }
            __syncthreads();
        }
        return;
    }

    // ---- moment stage: tile it - 1 (accumulators live only in these waves)
    f32x4 acc2[EM ? 2 : 1][EM ? NBLK : 1];
    f32x4 acc1[EM ? NB : 1];
    float s0r[2] = {0.0f, 0.0f};
    if constexpr (EM) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int q = 0; q < NBLK; ++q) acc2[c][q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) acc1[bb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    double ll = 0.0;
    __syncthreads();
    for (int it = 0; it <= nt; ++it) {
        if (it >= 1) {
            const int jt = it - 1;                  // tile of this stage
            const int64_t tt = t0 + jt;
            const uint16_t* xt = xr_s[jt % 3];
            const float(*gs)[kGS] = g_s[jt & 1];
            // base-2 LSE of the 256 points (4 per lane); gamma of components 2v, 2v + 1
#pragma unroll 1
            for (int m = 0; m < 4; ++m) {
                const int pt = lane + 64 * m;
                const int64_t p = tt * T + pt;
                const bool valid = p < n;
                float sv[KP];
                float M = -INFINITY;
#pragma unroll
                for (int k = 0; k < KP; ++k) {
                    sv[k] = gs[k][pt];
                    M = fmaxf(M, sv[k]);
                }
                const float Ms = M == -INFINITY ? 0.0f : M;
                float Z = 0.0f;
#pragma unroll
                for (int k = 0; k < KP; ++k) Z += fast_exp2(sv[k] - Ms);
                const float own = Ms + fast_log2(Z);
                // several groups: normalise with the merged LSE of all of them
                float lse2 = own;
                if constexpr (EXT) lse2 = valid ? ps.lse_in[p] * kLog2ef : 0.0f;
                if (v == 0 && valid) ll += (double)own;
                if constexpr (EM) {
                    const float lsafe = lse2 == -INFINITY ? INFINITY : lse2;
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        const float svc = gs[2 * v + c][pt];   // read again: sv[] is dead by now
                        const float gk = valid ? fast_exp2(svc - lsafe) : 0.0f;
                        s0r[c] += gk;
                        gp_s[v][c][pt] = __builtin_bit_cast(uint16_t, (_Float16)gk);   // the MFMA operand
                    }
                } else if (v == 0 && valid) {
                    if (ps.out_lse) ps.out_lse[p] = lse2 * kLn2f;
                    if (ps.out_arg) {
                        int a = 0;
#pragma unroll
                        for (int k = KP - 1; k >= 0; --k)
                            if (sv[k] == M) a = k;
                        ps.out_arg[p] = KP * ps.group + a;
                    }
                    if (ps.out_max) ps.out_max[p] = M;
                    if (ps.topm > 0) write_topm(sv, lse2, ps, p);
                }
            }
            if constexpr (EM) {
                // this wave's gamma row is read back by its own lanes: LDS operations of
                // one wave complete in order
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll 1
                for (int ks = 0; ks < T / 32; ++ks) {
                    const int pc = 32 * ks + 8 * g;   // this lane's 8 points of the K-step
                    uint4 xb[NB];
#pragma unroll
                    for (int bb = 0; bb < NB; ++bb) {
                        const int r0 = 32 * ks + 8 * g + (j >> 2), cu = 2 * bb + ((j & 3) >> 1);
                        const int co = 4 * (j & 1);   // halves within the 16-byte unit
                        const uint2 lo = tr16(&xt[xoff(r0, cu) + co]);
                        const uint2 hi = tr16(&xt[xoff(r0 + 4, cu) + co]);
                        xb[bb] = make_uint4(lo.x, lo.y, hi.x, hi.y);
                    }
                    {   // s1 of components 2v, 2v + 1: rows 0, 1 of gamma^T x (rows 2.. zero)
                        half8 ga = {0, 0, 0, 0, 0, 0, 0, 0};
                        if (j < 2) ga = *reinterpret_cast<const half8*>(&gp_s[v][j][pc]);
#pragma unroll
                        for (int bb = 0; bb < NB; ++bb)
                            acc1[bb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ga, __builtin_bit_cast(half8, xb[bb]),
                                                                            acc1[bb], 0, 0, 0);
                    }
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        __asm__ volatile("" ::: "memory");   // one component's operands at a time
                        const int k = 2 * v + c;
                        const half8 gh = *reinterpret_cast<const half8*>(&gp_s[v][c][pc]);
                        half8 yc[NB];
#pragma unroll
                        for (int bb = 0; bb < NB; ++bb) {
                            const half2v nm = __builtin_bit_cast(half2v, nm_s[k][16 * bb + j]);
                            yc[bb] = __builtin_bit_cast(half8, xb[bb]) +
                                     __builtin_shufflevector(nm, nm, 0, 1, 0, 1, 0, 1, 0, 1);
                        }
#pragma unroll
                        for (int ab = 0; ab < NB; ++ab) {
                            const half8 ya = yc[ab] * gh;   // gamma (x - mu_k)
#pragma unroll
                            for (int bb = 0; bb <= ab; ++bb)
                                acc2[c][blk_index(ab, bb)] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                    ya, yc[bb], acc2[c][blk_index(ab, bb)], 0, 0, 0);
                        }
                    }
                }
            }
        }
        __syncthreads();
    }

    // ---- epilogue: per-workgroup partials [KP][1 + D + D(D+1)/2], one writer each
    if constexpr (EM) {
        if (!p1) {
            const int ncolp = 1 + d + d * (d + 1) / 2;
            float* dst = part + (int64_t)b * KP * ncolp;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                float sv0 = s0r[c];
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) sv0 += __shfl_xor(sv0, o);
                if (lane == 0) dst[(int64_t)(2 * v + c) * ncolp] = sv0;
            }
            if (g == 0) {
#pragma unroll
                for (int bb = 0; bb < NB; ++bb)
#pragma unroll
                    for (int r = 0; r < 2; ++r) {
                        const int dd = 16 * bb + j;
                        if (dd < d) dst[(int64_t)(2 * v + r) * ncolp + 1 + dd] = acc1[bb][r];
                    }
            }
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int k = 2 * v + c;
#pragma unroll
                for (int ab = 0; ab < NB; ++ab)
#pragma unroll
                    for (int bb = 0; bb <= ab; ++bb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int row = 16 * ab + 4 * g + r, col = 16 * bb + j;
                            if (row >= col && row < d)
                                dst[(int64_t)k * ncolp + 1 + d + tri_idx(row, col)] =
                                    acc2[c][blk_index(ab, bb)][r];
                        }
            }
        }
    }
    // LL: moment wave 0 holds it
    if (w == 4) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) ll += __shfl_xor(ll, o);
        if (lane == 0 && part_ll != nullptr) part_ll[b] = seg_first ? ll * kLn2 : part_ll[b] + ll * kLn2;
    }
}

// ---------------------------------------------------------------------------
// 64 < D <= 128 (padded to 128).  The whitening panel of one component (the
// 20 lower-triangle 32 x 32 blocks of W, hi and lo: 160 registers per lane)
// and its lower-triangle second moments (36 blocks of 16 x 16: 144 registers)
// fill most of the 512 registers a lane has at one wave per SIMD, so a wave
// holds one component at a time, and the point work of every EM iteration
// takes the two loops over the components ([LP-GMM] 3.2): an E-step launch per
// group of 16 (k_full_wide_e, below) writes the group's log-sum-exp per point
// (merged over the groups afterwards), then one statistics launch per quad of
// components (k_full_wide) normalises with the merged LSE and accumulates the
// statistics (the whitening is done twice).
//   Statistics launch: components 4 quad .. 4 quad + 3 of the group, one per
//   wave, the panel loaded once; after the whitening every thread turns the
//   four scores of its point into responsibilities, then wave w accumulates
//   the second moments of its component and the first moments of dimension
//   blocks 2w, 2w + 1 of all four.
namespace wide {
constexpr int DP = 128, NB = 8, NBLK = 36, NOB = 4, NKS = 8;
constexpr int NPR = 20;          // lower-triangle (out block, K step) pairs: K step <= 2 ob + 1
constexpr int kXR = DP + 8;      // halves per row of the row-major tile
constexpr int kGS = T + 4;
constexpr int NVL = 2 * NOB * NKS;   // panel vectors per lane and component in memory
__host__ __device__ constexpr int pair_of(int ob, int ks) { return ob * (ob + 1) + ks; }

// The whitening MFMAs from inline asm: the accumulator stays in VGPRs (in the
// statistics launch the compiler would give it AGPRs next to the resident
// second moments, and the vector unit would then copy it out for |z|^2); the
// statistics launch reads the hi half of the panel from VGPRs and the lo half
// from AGPRs.  The compiler sees no MFMA in
// an asm statement, so the wait states are written out: two before each (a
// vector-ALU write of an operand just before an MFMA) and `settle` (24) after
// the last one of a block, before any other instruction touches the
// accumulators (a 32x32x16 result needs 18 before a vector-ALU read); its
// "+v" operands make every later use depend on it.
__device__ __forceinline__ void mfma_vv(f32x16& d, const half8& a, const half8& b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_av(f32x16& d, const half8& a, const half8& b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(d) : "a"(a), "v"(b));
}
__device__ __forceinline__ void settle(f32x16& p, f32x16& q, f32x16& r, f32x16& u) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(p), "+v"(q), "+v"(r), "+v"(u));
}
__device__ __forceinline__ void settle2(f32x16& p, f32x16& q) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(p), "+v"(q));
}
}  // namespace wide

template <bool VEC>
__global__ __launch_bounds__(256, 1) void k_full_wide(
    const _Float16* __restrict__ x, int64_t n, int d, int64_t ldx, const uint4* __restrict__ wpk,
    const float* __restrict__ wbias, const float* __restrict__ muh, const float* __restrict__ cvec,
    const float* __restrict__ rscale, float* __restrict__ part, const FullPass ps, int64_t tlo,
    int64_t thi) {
    using namespace wide;
    constexpr int KC = 4;   // components of this launch
    const int kq = 4 * ps.quad;   // the first of them within the group
    __shared__ __attribute__((aligned(16))) uint32_t nm_s[KC][DP];   // (-mu, -mu) fp16 pairs
    __shared__ __attribute__((aligned(16))) float wb_s[KC][DP];              // -W mu
    __shared__ float cv_s[KC], hq_s[KC];
    __shared__ __attribute__((aligned(16))) float g_s[KC][kGS];              // scores, then gamma
    // the tile, row-major, in two buffers: the next tile is written into the
    // other one during the whitening of this one
    __shared__ __attribute__((aligned(16))) uint16_t xr_s[2][T][kXR];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, j = lane & 15;

    for (int i = tid; i < KC * DP; i += 256) {
        const uint32_t h = __builtin_bit_cast(uint16_t, (_Float16)(-muh[(kq + i / DP) * DP + i % DP]));
        nm_s[i / DP][i % DP] = h | (h << 16);
    }
    for (int i = tid; i < KC * DP; i += 256) wb_s[i / DP][i % DP] = -wbias[(kq + i / DP) * DP + i % DP];
    if (tid < KC) {
        const float rs = rscale[kq + tid];
        cv_s[tid] = cvec[kq + tid];
        hq_s[tid] = kHalfLog2e * rs * rs;   // |z|^2 = 2^-2e |W x - W mu|^2
    }

    const int G = gridDim.x;
    const int64_t tiles = thi - tlo;
    const int64_t tb = tiles / G, tr = tiles % G;
    const int b = blockIdx.x;
    const int64_t t0 = tlo + b * tb + (b < tr ? b : tr);
    const int64_t t1 = t0 + tb + (b < tr ? 1 : 0);

    // dimensions 8c..8c+7 of this thread's point of tile t, zero outside
    // [0, N) x [0, D); every load from an in-bounds address, masked afterwards
    auto load_col = [&](int64_t t, int c) __attribute__((always_inline)) {
        const int64_t p = t * T + tid;
        const bool valid = p < n;
        const _Float16* row = x + (valid ? p : 0) * ldx;
        if constexpr (VEC) {
            const int cmax = d / 8;
            const uint4 v = *reinterpret_cast<const uint4*>(row + 8 * (c < cmax ? c : 0));
            const uint32_t m = (valid && c < cmax) ? ~0u : 0u;
            return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
        } else {
            const uint16_t* rb = reinterpret_cast<const uint16_t*>(row);
            uint32_t wv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int i0 = 8 * c + 2 * q;
                const uint32_t lo = rb[i0 < d ? i0 : 0], hi = rb[i0 + 1 < d ? i0 + 1 : 0];
                wv[q] = (valid && i0 < d ? lo : 0u) | ((valid && i0 + 1 < d ? hi : 0u) << 16);
            }
            return make_uint4(wv[0], wv[1], wv[2], wv[3]);
        }
    };
    // the same in two halves, so that a load's wait comes only where its value
    // is stored: the raw 16 bytes (vector path; the element-wise path masks as
    // it assembles), then the mask
    auto load_raw = [&](int64_t t, int c) __attribute__((always_inline)) {
        if constexpr (VEC) {
            const int64_t p = t * T + tid;
            const _Float16* row = x + (p < n ? p : 0) * ldx;
            const int cmax = d / 8;
            return *reinterpret_cast<const uint4*>(row + 8 * (c < cmax ? c : 0));
        } else {
            return load_col(t, c);
        }
    };
    auto finish = [&](int64_t t, int c, uint4 v) __attribute__((always_inline)) {
        if constexpr (VEC) {
            const uint32_t m = (t * T + tid < n && c < d / 8) ? ~0u : 0u;
            return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
        } else {
            return v;
        }
    };
    // the lower-triangle blocks of component kg's panel (group-local index)
    auto load_panel = [&](int kg, half8 (&wv)[2][NPR]) __attribute__((always_inline)) {
#pragma unroll
        for (int hl = 0; hl < 2; ++hl)
#pragma unroll
            for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
                for (int ks = 0; ks <= 2 * ob + 1; ++ks)
                    wv[hl][pair_of(ob, ks)] = __builtin_bit_cast(
                        half8, wpk[((int64_t)kg * NVL + (hl * NOB + ob) * NKS + ks) * 64 + lane]);
    };
    // base-2 scores of launch component kl for points 32 st .. 32 st + 31 of
    // the tile into g_s[kl]: lane l holds point l % 32 and out dimensions
    // 32 ob + 8 (r / 4) + 4 (l / 32) + r % 4; the accumulators start from -W mu
    auto whiten_step = [&](int kl, const half8 (&wv)[2][NPR], int cur, int st, float cvk,
                           float hqk) __attribute__((always_inline)) {
        {
            f32x16 acc[NOB];
#pragma unroll
            for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[ob][r] = wb_s[kl][32 * ob + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const half8 xb = __builtin_bit_cast(
                    half8, *reinterpret_cast<const uint4*>(&xr_s[cur][32 * st + (lane & 31)][16 * ks + 8 * (lane >> 5)]));
#pragma unroll
                for (int ob = 0; ob < NOB; ++ob) {
                    if (ks > 2 * ob + 1) continue;   // above the diagonal: W is lower triangular
                    mfma_vv(acc[ob], wv[0][pair_of(ob, ks)], xb);
                    mfma_av(acc[ob], wv[1][pair_of(ob, ks)], xb);
                }
            }
            settle(acc[0], acc[1], acc[2], acc[3]);
            float qp[4] = {0.0f, 0.0f, 0.0f, 0.0f};   // four chains: |z|^2 waits on no long chain
#pragma unroll
            for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
                for (int r = 0; r < 16; ++r) qp[r & 3] = fmaf(acc[ob][r], acc[ob][r], qp[r & 3]);
            const float q = halves_sum((qp[0] + qp[1]) + (qp[2] + qp[3]));
            if (lane < 32) g_s[kl][32 * st + lane] = cvk - hqk * q;
        }
    };

    float s0acc[4] = {};
    f32x4 acc2[NBLK];
    f32x4 acc1[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int q = 0; q < NBLK; ++q) acc2[q] = f32x4{0.f, 0.f, 0.f, 0.f};

    half8 wv[2][NPR];
    {
        load_panel(kq + w, wv);
        // wait for the panel here, once: otherwise the wait inserted before its
        // first use inside the tile loop stays in the loop and also waits for
        // the loads of the next tile issued just before
#pragma unroll
        for (int i = 0; i < NPR; ++i) asm volatile("" : : "v"(wv[0][i]), "a"(wv[1][i]));
        if (t0 < t1) {
#pragma unroll
            for (int c = 0; c < DP / 8; ++c) *reinterpret_cast<uint4*>(&xr_s[0][tid][8 * c]) = load_col(t0, c);
        }
    }
    for (int64_t t = t0; t < t1; ++t) {
        const int64_t p = t * T + tid;
        const bool valid = p < n;
        const int cur = (int)((t - t0) & 1);
        __syncthreads();   // the previous tile is done with g_s (and its own buffer)
        {
            // the next tile goes to the other buffer (it held tile t - 1) two
            // 16-byte columns per whitening step, each stored three steps after
            // its loads were issued: 32 registers in flight instead of 64
            // (after the last tile: tile t again, into a buffer no one reads; the
            // loads are not conditional, so each one's wait stays where it is stored)
            const int64_t tn = t + 1 < t1 ? t + 1 : t;
            const float cvk = cv_s[w], hqk = hq_s[w];
            uint4 nx[4][2];
#pragma unroll
            for (int st = 0; st < T / 32; ++st) {
                nx[st % 4][0] = load_raw(tn, 2 * st);
                nx[st % 4][1] = load_raw(tn, 2 * st + 1);
                if (st >= 3) {
                    const int c = 2 * (st - 3);
                    *reinterpret_cast<uint4*>(&xr_s[cur ^ 1][tid][8 * c]) = finish(tn, c, nx[(st - 3) % 4][0]);
                    *reinterpret_cast<uint4*>(&xr_s[cur ^ 1][tid][8 * c + 8]) = finish(tn, c + 1, nx[(st - 3) % 4][1]);
                }
                whiten_step(w, wv, cur, st, cvk, hqk);
            }
#pragma unroll
            for (int st = T / 32; st < T / 32 + 3; ++st) {
                const int c = 2 * (st - 3);
                *reinterpret_cast<uint4*>(&xr_s[cur ^ 1][tid][8 * c]) = finish(tn, c, nx[(st - 3) % 4][0]);
                *reinterpret_cast<uint4*>(&xr_s[cur ^ 1][tid][8 * c + 8]) = finish(tn, c + 1, nx[(st - 3) % 4][1]);
            }
        }
        __syncthreads();

        {   // responsibilities from the merged LSE of all groups
            const float lse2 = valid ? ps.lse_in[p] * kLog2ef : 0.0f;
            const float lsafe = lse2 == -INFINITY ? INFINITY : lse2;   // no live component
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float gk = valid ? fast_exp2(g_s[k][tid] - lsafe) : 0.0f;
                s0acc[k] += gk;
                g_s[k][tid] = gk;
            }
        }

        {
            __syncthreads();
#pragma unroll 1
            for (int ks = 0; ks < T / 32; ++ks) {
                const int pc = 32 * ks + 8 * g;   // this lane's 8 points of the K step
                // x of points pc..pc+7, dimension 16 bb + j: two transposed reads of the tile
                uint4 xb[NB];
#pragma unroll
                for (int bb = 0; bb < NB; ++bb) {
                    const uint16_t* src = &xr_s[cur][32 * ks + 8 * g + (j >> 2)][16 * bb + 4 * (j & 3)];
                    const uint2 lo = tr16(src), hi = tr16(src + 4 * kXR);
                    xb[bb] = make_uint4(lo.x, lo.y, hi.x, hi.y);
                }
                {   // s1 += gamma^T x: rows 0..3 the four components, dims 16 bb + j (bb = 2w, 2w + 1)
                    half8 ga = {};
                    if (j < 4) {
                        const float4 g0 = *reinterpret_cast<const float4*>(&g_s[j][pc]);
                        const float4 g1 = *reinterpret_cast<const float4*>(&g_s[j][pc + 4]);
                        ga = half8{(_Float16)g0.x, (_Float16)g0.y, (_Float16)g0.z, (_Float16)g0.w,
                                   (_Float16)g1.x, (_Float16)g1.y, (_Float16)g1.z, (_Float16)g1.w};
                    }
#pragma unroll
                    for (int h = 0; h < 2; ++h) {   // read again: xb is not indexed by the wave
                        const uint16_t* src = &xr_s[cur][32 * ks + 8 * g + (j >> 2)][16 * (2 * w + h) + 4 * (j & 3)];
                        const uint2 lo = tr16(src), hi = tr16(src + 4 * kXR);
                        acc1[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            ga, __builtin_bit_cast(half8, make_uint4(lo.x, lo.y, hi.x, hi.y)), acc1[h], 0, 0, 0);
                    }
                }
                const float4 g0 = *reinterpret_cast<const float4*>(&g_s[w][pc]);
                const float4 g1 = *reinterpret_cast<const float4*>(&g_s[w][pc + 4]);
                const half8 gh = {(_Float16)g0.x, (_Float16)g0.y, (_Float16)g0.z, (_Float16)g0.w,
                                  (_Float16)g1.x, (_Float16)g1.y, (_Float16)g1.z, (_Float16)g1.w};
                half8 yc[NB];
#pragma unroll
                for (int bb = 0; bb < NB; ++bb) {
                    const half2v nm = __builtin_bit_cast(half2v, nm_s[w][16 * bb + j]);
                    yc[bb] = __builtin_bit_cast(half8, xb[bb]) + __builtin_shufflevector(nm, nm, 0, 1, 0, 1, 0, 1, 0, 1);
                }
#pragma unroll
                for (int ab = 0; ab < NB; ++ab) {
                    const half8 ya = yc[ab] * gh;   // gamma (x - mu_k)
#pragma unroll
                    for (int bb = 0; bb <= ab; ++bb)
                        acc2[blk_index(ab, bb)] =
                            __builtin_amdgcn_mfma_f32_16x16x32_f16(ya, yc[bb], acc2[blk_index(ab, bb)], 0, 0, 0);
                }
            }
        }
    }

    __syncthreads();
    {
        // rows kq..kq+3 of this workgroup's partial slot [KP][1 + D + D(D+1)/2]
        const int ncolp = 1 + d + d * (d + 1) / 2;
        float* dst = part + (int64_t)b * KP * ncolp;
#pragma unroll
        for (int k = 0; k < 4; ++k) g_s[k][tid] = s0acc[k];
        __syncthreads();
        if (tid < 4) {
            double s = 0.0;
            for (int i = 0; i < T; ++i) s += (double)g_s[tid][i];
            dst[(int64_t)(kq + tid) * ncolp] = (float)s;
        }
        if (g == 0) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int dd = 16 * (2 * w + h) + j;
                    if (dd < d) dst[(int64_t)(kq + r) * ncolp + 1 + dd] = acc1[h][r];
                }
        }
#pragma unroll
        for (int ab = 0; ab < NB; ++ab)
#pragma unroll
            for (int bb = 0; bb <= ab; ++bb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * ab + 4 * g + r, col = 16 * bb + j;
                    if (row >= col && row < d)
                        dst[(int64_t)(kq + w) * ncolp + 1 + d + tri_idx(row, col)] = acc2[blk_index(ab, bb)][r];
                }
    }
}

// E-step launch for 64 < D <= 128 over a group of 16 components: eight waves,
// two per SIMD.  Wave w takes components 4 (w / 2) .. + 3 in turn and, of
// each, half of the lower-triangle output blocks of W (x - mu): blocks 0 and 3
// (10 of the 20 (block, K step) pairs) for even w, blocks 1 and 2 (the other
// 10) for odd w, so a wave holds half a panel (80 registers) and the other
// wave on its SIMD fills the gaps of its own (the panel loads of each
// component, |z|^2 after each 32-point block).  The two halves of |z|^2 meet
// in LDS; every thread of the first four waves then forms its point's
// log-sum-exp and per-point outputs as k_full_fused does.
namespace wide_e {
constexpr int kThreads = 512;
constexpr int NP = 10;   // (block, K step) pairs per half
// pair p of half h: output block and K step
__host__ __device__ constexpr int blk(int h, int p) { return h == 0 ? (p < 2 ? 0 : 3) : (p < 4 ? 1 : 2); }
__host__ __device__ constexpr int kst(int h, int p) { return h == 0 ? (p < 2 ? p : p - 2) : (p < 4 ? p : p - 4); }
}  // namespace wide_e

template <bool VEC>
__global__ __launch_bounds__(wide_e::kThreads, 1) void k_full_wide_e(
    const _Float16* __restrict__ x, int64_t n, int d, int64_t ldx, const uint4* __restrict__ wpk,
    const float* __restrict__ wbias, const float* __restrict__ cvec, const float* __restrict__ rscale,
    double* __restrict__ part_ll, const FullPass ps, int64_t tlo, int64_t thi, int seg_first) {
    using namespace wide;
    using wide_e::NP;
    __shared__ __attribute__((aligned(16))) uint16_t xr_s[T][kXR];   // the tile, row-major
    __shared__ __attribute__((aligned(16))) float gq_s[2][KP][kGS];  // the two halves of |z|^2
    __shared__ __attribute__((aligned(16))) float wb_s[KP][DP];      // -W mu
    __shared__ float cv_s[KP], hq_s[KP];
    __shared__ double red[wide_e::kThreads];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = w & 1, kc = 4 * (w >> 1);
    for (int i = tid; i < KP * DP; i += wide_e::kThreads) wb_s[i / DP][i % DP] = -wbias[i];
    if (tid < KP) {
        const float rs = rscale[tid];
        cv_s[tid] = cvec[tid];
        hq_s[tid] = kHalfLog2e * rs * rs;   // |z|^2 = 2^-2e |W x - W mu|^2
    }

    const int G = gridDim.x;
    const int64_t tiles = thi - tlo;
    const int64_t tb = tiles / G, tr = tiles % G;
    const int b = blockIdx.x;
    const int64_t t0 = tlo + b * tb + (b < tr ? b : tr);
    const int64_t t1 = t0 + tb + (b < tr ? 1 : 0);

    // staging: thread tid holds half a row of the next tile, point tid / 2 and
    // 16-byte columns 8 (tid % 2) .. + 7, loaded raw and masked when stored
    const int sp = tid >> 1, sc = 8 * (tid & 1);
    uint4 xv[8];
    auto load_half = [&](int64_t t) __attribute__((always_inline)) {
        const int64_t p = t * T + sp;
        const _Float16* row = x + (p < n ? p : 0) * ldx;
        if constexpr (VEC) {
            const int cmax = d / 8;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int c = sc + i;
                xv[i] = *reinterpret_cast<const uint4*>(row + 8 * (c < cmax ? c : 0));
            }
        } else {
            const bool valid = p < n;
            const uint16_t* rb = reinterpret_cast<const uint16_t*>(row);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                uint32_t wq[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int i0 = 8 * (sc + i) + 2 * q;
                    const uint32_t lo = rb[i0 < d ? i0 : 0], hi = rb[i0 + 1 < d ? i0 + 1 : 0];
                    wq[q] = (valid && i0 < d ? lo : 0u) | ((valid && i0 + 1 < d ? hi : 0u) << 16);
                }
                xv[i] = make_uint4(wq[0], wq[1], wq[2], wq[3]);
            }
        }
    };
    auto store_half = [&](int64_t t) __attribute__((always_inline)) {
        const bool valid = t * T + sp < n;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint4 v = xv[i];
            if constexpr (VEC) {
                const uint32_t m = (valid && sc + i < d / 8) ? ~0u : 0u;
                v = make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
            }
            *reinterpret_cast<uint4*>(&xr_s[sp][8 * (sc + i)]) = v;
        }
    };

    double ll = 0.0;
    if (t0 < t1) load_half(t0);
    for (int64_t t = t0; t < t1; ++t) {
        __syncthreads();   // the previous tile is done with xr_s / gq_s
        store_half(t);
        __syncthreads();
        if (t + 1 < t1) load_half(t + 1);   // the next tile, behind this one's work
        // the half's pairs as constants: one copy of the loop per half
        auto whiten = [&](auto half) __attribute__((always_inline)) {
            constexpr int H = decltype(half)::value;
            constexpr int OB0 = H == 0 ? 0 : 1, OB1 = H == 0 ? 3 : 2;   // its two blocks
            constexpr int N0 = 2 * OB0 + 2;   // pairs (K steps) of block OB0; OB1 takes the rest
#pragma unroll 1
            for (int kk = 0; kk < 4; ++kk) {
                const int k = kc + kk;
                half8 wv[2][NP];   // this half of component k's panel
#pragma unroll
                for (int hl = 0; hl < 2; ++hl)
#pragma unroll
                    for (int pp = 0; pp < NP; ++pp)
                        wv[hl][pp] = __builtin_bit_cast(
                            half8, wpk[((int64_t)k * NVL + (hl * NOB + wide_e::blk(H, pp)) * NKS + wide_e::kst(H, pp)) * 64 + lane]);
#pragma unroll 1
                for (int st = 0; st < T / 32; ++st) {
                    f32x16 acc[2];
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int o = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                        acc[0][r] = wb_s[k][32 * OB0 + o];
                        acc[1][r] = wb_s[k][32 * OB1 + o];
                    }
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) {
                        const half8 xb = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(
                            &xr_s[32 * st + (lane & 31)][16 * ks + 8 * (lane >> 5)]));
                        if (ks < N0) {
                            mfma_vv(acc[0], wv[0][ks], xb);
                            mfma_vv(acc[0], wv[1][ks], xb);
                        }
                        if (ks <= 2 * OB1 + 1) {
                            mfma_vv(acc[1], wv[0][N0 + ks], xb);
                            mfma_vv(acc[1], wv[1][N0 + ks], xb);
                        }
                    }
                    settle2(acc[0], acc[1]);
                    float qp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        qp[r & 3] = fmaf(acc[0][r], acc[0][r], qp[r & 3]);
                        qp[r & 3] = fmaf(acc[1][r], acc[1][r], qp[r & 3]);
                    }
                    const float q = halves_sum((qp[0] + qp[1]) + (qp[2] + qp[3]));
                    if (lane < 32) gq_s[H][k][32 * st + lane] = q;
                }
            }
        };
        if (h == 0) whiten(std::integral_constant<int, 0>{});
        else whiten(std::integral_constant<int, 1>{});
        __syncthreads();

        // ---- base-2 log-sum-exp of the group, per-point outputs
        if (tid < T) {
            const int64_t p = t * T + tid;
            const bool valid = p < n;
            float sv[KP];
            float M = -INFINITY;
#pragma unroll
            for (int k = 0; k < KP; ++k) {
                sv[k] = cv_s[k] - hq_s[k] * (gq_s[0][k][tid] + gq_s[1][k][tid]);
                M = fmaxf(M, sv[k]);
            }
            const float Ms = M == -INFINITY ? 0.0f : M;
            float Z = 0.0f;
#pragma unroll
            for (int k = 0; k < KP; ++k) Z += fast_exp2(sv[k] - Ms);
            const float own = Ms + fast_log2(Z);
            const float lse2 = ps.lse_in != nullptr ? (valid ? ps.lse_in[p] * kLog2ef : 0.0f) : own;
            if (valid) {
                ll += (double)own;
                if (ps.out_lse) ps.out_lse[p] = lse2 * kLn2f;
                if (ps.out_arg) {
                    int a = 0;
#pragma unroll
                    for (int k = KP - 1; k >= 0; --k)
                        if (sv[k] == M) a = k;
                    ps.out_arg[p] = KP * ps.group + a;
                }
                if (ps.out_max) ps.out_max[p] = M;
                if (ps.topm > 0) write_topm(sv, lse2, ps, p);
            }
        }
    }

    red[tid] = ll;
    __syncthreads();
    for (int s2 = wide_e::kThreads / 2; s2 > 0; s2 >>= 1) {
        if (tid < s2) red[tid] += red[tid + s2];
        __syncthreads();
    }
    if (tid == 0 && part_ll != nullptr) part_ll[b] = seg_first ? red[0] * kLn2 : part_ll[b] + red[0] * kLn2;
}

// Group g's slice of the per-component arrays and partial slots.
struct FullGroupPtrs {
    const uint4* wpk;
    const float *wbias, *muh, *cvec, *rscale;
    float* part;
};
template <int DP>
FullGroupPtrs group_ptrs(const Plan& p, const FullWs& w, int g) {
    constexpr int NV = FullShape<DP>::kNV;
    FullGroupPtrs q;
    q.wpk = w.wpk + (size_t)g * KP * NV * 64;
    q.wbias = w.wbias + (size_t)g * KP * full_dpo(DP);
    q.muh = w.muh + (size_t)g * KP * DP;
    q.cvec = w.cvec + (size_t)g * KP;
    q.rscale = w.rscale + (size_t)g * KP;
    q.part = w.part + (size_t)g * w.slots * KP * full_ncolp(p.d);
    return q;
}

template <int DP, bool VEC>
hipError_t launch_dv(const Plan& p, const FullWs& w, const void* x, bool em, int grid,
                     const FullPass& ps, double* pll, int64_t tlo, int64_t thi, int seg_first,
                     hipStream_t s) {
    const FullGroupPtrs q = group_ptrs<DP>(p, w, ps.group);
    if (em)
        hipLaunchKernelGGL((k_full_fused<DP, true, VEC>), dim3(grid), dim3(256), 0, s,
                           (const _Float16*)x, p.n, (int)p.d, p.ldx, (int)p.k, q.wpk, q.wbias, q.muh,
                           q.cvec, q.rscale, q.part, pll, ps, tlo, thi, seg_first);
    else
        hipLaunchKernelGGL((k_full_fused<DP, false, VEC>), dim3(grid), dim3(256), 0, s,
                           (const _Float16*)x, p.n, (int)p.d, p.ldx, (int)p.k, q.wpk, q.wbias, q.muh,
                           q.cvec, q.rscale, q.part, pll, ps, tlo, thi, seg_first);
    return hipGetLastError();
}

template <int DP>
hipError_t launch_dp(const Plan& p, const FullWs& w, const void* x, bool em, int grid,
                     const FullPass& ps, int64_t tlo, int64_t thi, int seg_first, hipStream_t s) {
    const bool vec = (uintptr_t)x % 16 == 0 && p.ldx % 8 == 0 && p.d % 8 == 0;
    // LL partials only from a group that is the only one (several: the merge sums the LL)
    double* pll = w.lse_pass ? nullptr : w.part_ll;
    if (DP == 64 && vec) {   // the pipelined kernel
        const FullGroupPtrs q = group_ptrs<64>(p, w, ps.group);
#define FULL_PIPE(EM_, EXT_)                                                                     \
    hipLaunchKernelGGL((k_full_pipe<EM_, EXT_>), dim3(grid), dim3(pipe::kThreads), 0, s,          \
                       (const _Float16*)x, p.n, (int)p.d, p.ldx, (int)p.k, q.wpk, q.wbias, q.muh, \
                       q.cvec, q.rscale, q.part, pll, ps, tlo, thi, seg_first)
        const bool ext = ps.lse_in != nullptr;
        if (em && ext) FULL_PIPE(true, true);
        else if (em) FULL_PIPE(true, false);
        else if (ext) FULL_PIPE(false, true);
        else FULL_PIPE(false, false);
#undef FULL_PIPE
        return hipGetLastError();
    }
    return vec ? launch_dv<DP, true>(p, w, x, em, grid, ps, pll, tlo, thi, seg_first, s)
               : launch_dv<DP, false>(p, w, x, em, grid, ps, pll, tlo, thi, seg_first, s);
}

// D <= 128: E-step launches over a group of 16, E+M launches over quad ps.quad
// of it (normalised with ps.lse_in, the merged LSE; the LL comes from the merge)
hipError_t launch_wide(const Plan& p, const FullWs& w, const void* x, bool em, int grid,
                       const FullPass& ps, int64_t tlo, int64_t thi, int seg_first, hipStream_t s) {
    if (em && ps.lse_in == nullptr) return hipErrorInvalidValue;
    const bool vec = (uintptr_t)x % 16 == 0 && p.ldx % 8 == 0 && p.d % 8 == 0;
    const FullGroupPtrs q = group_ptrs<wide::DP>(p, w, ps.group);
    double* pll = (!em && !w.lse_pass) ? w.part_ll : nullptr;
#define FULL_WIDE(VEC_)                                                                          \
    hipLaunchKernelGGL((k_full_wide<VEC_>), dim3(grid), dim3(256), 0, s, (const _Float16*)x, p.n, \
                       (int)p.d, p.ldx, q.wpk, q.wbias, q.muh, q.cvec, q.rscale, q.part, ps, tlo, thi)
#define FULL_WIDE_E(VEC_)                                                                        \
    hipLaunchKernelGGL((k_full_wide_e<VEC_>), dim3(grid), dim3(wide_e::kThreads), 0, s,          \
                       (const _Float16*)x, p.n, (int)p.d, p.ldx, q.wpk, q.wbias, q.cvec, q.rscale, \
                       pll, ps, tlo, thi, seg_first)
    if (em && vec) FULL_WIDE(true);
    else if (em) FULL_WIDE(false);
    else if (vec) FULL_WIDE_E(true);
    else FULL_WIDE_E(false);
#undef FULL_WIDE
#undef FULL_WIDE_E
    return hipGetLastError();
}

}  // namespace

int full_grid(const Plan& p) {
    const int64_t tiles = (p.n + kFullT - 1) / kFullT;
    int64_t g = device_cu_count();
    if (g > p.p_max) g = p.p_max;
    if (g > tiles) g = tiles;
    return (int)(g < 1 ? 1 : g);
}

hipError_t full_launch_fused(const Plan& p, const FullWs& w, const void* x, bool em, int grid,
                             const FullPass& ps, int64_t tlo, int64_t thi, int seg_first,
                             hipStream_t s) {
    switch (p.dp) {
        case 16: return launch_dp<16>(p, w, x, em, grid, ps, tlo, thi, seg_first, s);
        case 32: return launch_dp<32>(p, w, x, em, grid, ps, tlo, thi, seg_first, s);
        case 64: return launch_dp<64>(p, w, x, em, grid, ps, tlo, thi, seg_first, s);
        case 128: return launch_wide(p, w, x, em, grid, ps, tlo, thi, seg_first, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gmm
