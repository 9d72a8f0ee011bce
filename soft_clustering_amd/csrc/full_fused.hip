// Full-covariance Gaussian mixture, X stored in fp16: fused E-step + M-step
// statistics, one pass over X, no N x K matrix in memory.
//
// Density ([LP-GMM] 1.2, route 2): d^2 = |z|^2 with L z = x - mu solved by
// forward substitution (no inverse), L the ridged Cholesky factor stored in
// fp16 ([LP-GMM] 2.1 storage plan, 4.1 ridge); log|C| = 2 sum log L_ii.  The
// solve and every exp / log / normaliser run in fp32 ([LP-GMM] 1.3 first
// boundary): the fp16 entries of L feed v_fma_mix_f32 directly.
// Statistics ([Flash-GMM] Method, s0 / s1 / sum gamma x x^T on chip): s1 =
// gamma^T X and the centred second moment sum_n gamma_nk (x_n - mu_k)
// (x_n - mu_k)^T (lower-triangle 16 x 16 blocks) on fp16 MFMA
// (v_mfma_f32_16x16x32_f16) with fp32 accumulation; the M-step turns them into
// raw moments and the new covariance in fp64.
//
// Work split: a workgroup of 256 threads takes 256-point tiles.  Phase 1: each
// thread solves its own point against every component (L of all components
// staged once in LDS, broadcast reads), forms the base-2 log-sum-exp and the
// responsibilities in registers, and writes gamma^T and x^T for the tile to
// LDS.  Phase 2 (E+M only): wave w accumulates the second moments of
// components 4w..4w+3 and the first moments of dimension block w over the
// tile.  Two barriers per tile.

#include "full_internal.h"

namespace gmm {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

constexpr int KP = kFullKP;
constexpr int T = kFullT;
constexpr float kLn2f = 0.69314718055994530942f;
constexpr float kHalfLog2e = 0.72134752044448170368f;   // log2(e) / 2

template <int DP>
struct FullShape {
    static constexpr int kLH = full_l_halves(DP);       // halves of packed L per component
    static constexpr int kNB = DP / 16;                  // 16-dim blocks
    static constexpr int kNBlk = kNB * (kNB + 1) / 2;    // lower-triangle 16 x 16 blocks
    static constexpr int kXT = T + 8;                    // halves per x^T row
};

__device__ __forceinline__ int blk_index(int ab, int bb) { return ab * (ab + 1) / 2 + bb; }

template <int DP, bool EM>
__global__ __launch_bounds__(256, 1) void k_full_fused(
    const _Float16* __restrict__ x, int64_t n, int d, int64_t ldx, int k_real, int vec,
    const uint16_t* __restrict__ lpk, const float* __restrict__ pdiag, const float* __restrict__ muh,
    const float* __restrict__ cvec, const float* __restrict__ rscale, double* __restrict__ part,
    double* __restrict__ part_ll, float* __restrict__ out_lse, int* __restrict__ out_arg) {
    using Sh = FullShape<DP>;
    constexpr int NB = Sh::kNB, NBLK = Sh::kNBlk;
    __shared__ __attribute__((aligned(16))) uint16_t l_s[KP * Sh::kLH];
    __shared__ __attribute__((aligned(16))) float pd_s[KP][DP];
    __shared__ __attribute__((aligned(16))) float ms_s[KP][DP];      // mu * 2^-e_k
    __shared__ __attribute__((aligned(16))) uint16_t mh_s[KP][DP];   // fp16 mu
    __shared__ float cv_s[KP], rs_s[KP];
    __shared__ __attribute__((aligned(16))) float g_s[KP][T];        // scores, then gamma
    __shared__ __attribute__((aligned(16))) uint16_t xt_s[EM ? DP : 1][Sh::kXT];
    __shared__ double red[256];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, j = lane & 15;

    // ---- stage the prepared parameters of all components
    {
        const uint4* src = reinterpret_cast<const uint4*>(lpk);
        uint4* dst = reinterpret_cast<uint4*>(l_s);
        for (int i = tid; i < KP * Sh::kLH / 8; i += 256) dst[i] = src[i];
        for (int i = tid; i < KP * DP; i += 256) {
            const int k = i / DP, dd = i % DP;
            pd_s[k][dd] = pdiag[i];
            const float m = muh[i];
            ms_s[k][dd] = m * rscale[k];
            mh_s[k][dd] = __builtin_bit_cast(uint16_t, (_Float16)m);
        }
        if (tid < KP) {
            cv_s[tid] = cvec[tid];
            rs_s[tid] = rscale[tid];
        }
    }

    const int G = gridDim.x;
    const int64_t tiles = (n + T - 1) / T;
    const int64_t tb = tiles / G, tr = tiles % G;
    const int b = blockIdx.x;
    const int64_t t0 = b * tb + (b < tr ? b : tr);
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

    for (int64_t t = t0; t < t1; ++t) {
        const int64_t p = t * T + tid;
        const bool valid = p < n;
        // ---- load this thread's point (fp16 -> fp32), zero outside [0, N) x [0, D)
        float xf[DP];
        {
            const _Float16* row = x + (valid ? p : 0) * ldx;
            if (vec) {
#pragma unroll
                for (int c = 0; c < DP / 8; ++c) {
                    uint4 v = make_uint4(0, 0, 0, 0);
                    if (8 * c < d) v = *reinterpret_cast<const uint4*>(row + 8 * c);
                    const half8 h = __builtin_bit_cast(half8, v);
#pragma unroll
                    for (int e = 0; e < 8; ++e) xf[8 * c + e] = valid ? (float)h[e] : 0.0f;
                }
            } else {
#pragma unroll
                for (int i = 0; i < DP; ++i) xf[i] = (valid && i < d) ? (float)row[i] : 0.0f;
            }
        }
        __syncthreads();   // the previous tile's phase 2 is done with g_s / xt_s

        // ---- phase 1: forward solve against every component (fp32)
        for (int k = 0; k < KP; ++k) {
            const uint16_t* Lk = l_s + k * Sh::kLH;
            const float s = rs_s[k];
            float z[DP];
            float q0 = 0.f, q1 = 0.f, q2 = 0.f, q3 = 0.f;   // |z|^2 partial sums
#pragma unroll
            for (int i = 0; i < DP; ++i) {
                const float r = fmaf(xf[i], s, -ms_s[k][i]);
                float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
                for (int jb = 0; jb < DP / 8; ++jb) {   // constant trip count: unrolls fully
                    if (8 * jb >= i) continue;
                    const half8 lh = __builtin_bit_cast(
                        half8, *reinterpret_cast<const uint4*>(Lk + full_row_off(i) + 8 * jb));
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int jj = 8 * jb + e;
                        if (jj < i) {
                            const float lv = (float)lh[e];   // v_fma_mix_f32
                            if ((e & 3) == 0) a0 = fmaf(lv, z[jj], a0);
                            else if ((e & 3) == 1) a1 = fmaf(lv, z[jj], a1);
                            else if ((e & 3) == 2) a2 = fmaf(lv, z[jj], a2);
                            else a3 = fmaf(lv, z[jj], a3);
                        }
                    }
                }
                z[i] = (r - ((a0 + a1) + (a2 + a3))) * pd_s[k][i];
                if ((i & 3) == 0) q0 = fmaf(z[i], z[i], q0);
                else if ((i & 3) == 1) q1 = fmaf(z[i], z[i], q1);
                else if ((i & 3) == 2) q2 = fmaf(z[i], z[i], q2);
                else q3 = fmaf(z[i], z[i], q3);
            }
            g_s[k][tid] = cv_s[k] - kHalfLog2e * ((q0 + q1) + (q2 + q3));
        }

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
            const float lse2 = Ms + fast_log2(Z);
            if (valid) ll += (double)lse2;
            if constexpr (EM) {
                const float lsafe = lse2 == -INFINITY ? INFINITY : lse2;   // no live component
#pragma unroll
                for (int k = 0; k < KP; ++k) {
                    const float gk = valid ? fast_exp2(sv[k] - lsafe) : 0.0f;
                    s0acc[k] += gk;
                    g_s[k][tid] = gk;
                }
#pragma unroll
                for (int i = 0; i < DP; ++i) xt_s[i][tid] = __builtin_bit_cast(uint16_t, (_Float16)xf[i]);
            } else if (valid) {
                if (out_lse) out_lse[p] = lse2 * kLn2f;
                if (out_arg) {
                    int a = 0;
#pragma unroll
                    for (int k = KP - 1; k >= 0; --k)
                        if (sv[k] == M) a = k;
                    out_arg[p] = a;
                }
            }
        }

        if constexpr (EM) {
            __syncthreads();
            // ---- phase 2: second moments of components 4w..4w+3, first moments of dims block w
#pragma unroll 1
            for (int ks = 0; ks < T / 32; ++ks) {
                const int pc = 32 * ks + 8 * g;   // this lane's 8 points of the K-step
                uint4 xb[NB];
#pragma unroll
                for (int bb = 0; bb < NB; ++bb)
                    xb[bb] = *reinterpret_cast<const uint4*>(&xt_s[16 * bb + j][pc]);
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
                        const _Float16 m = __builtin_bit_cast(_Float16, mh_s[k][16 * bb + j]);
                        const half8 xv = __builtin_bit_cast(half8, xb[bb]);
                        yc[bb] = xv - m;      // (x - mu_k) in fp16, packed
                        ya[bb] = yc[bb] * gh; // gamma (x - mu_k)
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
        double* dst = part + (int64_t)b * KP * ncolp;
#pragma unroll
        for (int k = 0; k < KP; ++k) g_s[k][tid] = s0acc[k];
        __syncthreads();
        if (tid < KP) {
            double s = 0.0;
            for (int i = 0; i < T; ++i) s += (double)g_s[tid][i];
            dst[(int64_t)tid * ncolp] = s;
        }
        if (w < NB) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int k = 4 * g + r, dd = 16 * w + j;
                if (dd < d) dst[(int64_t)k * ncolp + 1 + dd] = (double)acc1[r];
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
                                (double)acc2[kk][blk_index(ab, bb)][r];
                    }
        }
    }
    red[tid] = ll;
    __syncthreads();
    for (int s2 = 128; s2 > 0; s2 >>= 1) {
        if (tid < s2) red[tid] += red[tid + s2];
        __syncthreads();
    }
    if (tid == 0) part_ll[b] = red[0] * kLn2;
}

template <int DP>
hipError_t launch_dp(const Plan& p, const FullWs& w, const void* x, bool em, int grid, float* lse,
                     int* arg, hipStream_t s) {
    const int vec = ((uintptr_t)x % 16 == 0 && p.ldx % 8 == 0 && p.d % 8 == 0) ? 1 : 0;
    if (em)
        hipLaunchKernelGGL((k_full_fused<DP, true>), dim3(grid), dim3(256), 0, s, (const _Float16*)x,
                           p.n, (int)p.d, p.ldx, (int)p.k, vec, w.lpk, w.pdiag, w.muh, w.cvec,
                           w.rscale, w.part, w.part_ll, (float*)nullptr, (int*)nullptr);
    else
        hipLaunchKernelGGL((k_full_fused<DP, false>), dim3(grid), dim3(256), 0, s, (const _Float16*)x,
                           p.n, (int)p.d, p.ldx, (int)p.k, vec, w.lpk, w.pdiag, w.muh, w.cvec,
                           w.rscale, w.part, w.part_ll, lse, arg);
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
                             float* lse, int* arg, hipStream_t s) {
    switch (p.dp) {
        case 16: return launch_dp<16>(p, w, x, em, grid, lse, arg, s);
        case 32: return launch_dp<32>(p, w, x, em, grid, lse, arg, s);
        case 64: return launch_dp<64>(p, w, x, em, grid, lse, arg, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gmm
