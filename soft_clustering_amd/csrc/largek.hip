// Large-K Gaussian mixtures (isotropic or diagonal covariance, X stored in
// bf16 or fp16): fused E-step + M-step statistics on fp16 MFMA
// (v_mfma_f32_16x16x32_f16, fp32 accumulation), fp32 softmax.
//
// Method: [Flash-GMM] Method, fused E-M step (tiles of X, softmax over K on
// chip, s0 / s1 / s2 accumulated without writing the N x K matrix).  When K
// spans several workgroups the log-sum-exp takes two sweeps, as in
// [LP-GMM] 3.2 (first loop over the components: maximum and normaliser;
// second loop: posteriors, distances recomputed).  exp, log, the normalisers
// and every statistic are fp32 ([LP-GMM] 1.3 first boundary, 2.1).
//
// Scores, base 2, from the expanded quadratic form ([LP-GMM] 3.1 panel):
//   y'_d = (x_d - c_d) s_d   (c: a centre, s_d = 2^-e_d: a power-of-two scale
//                             that keeps y' and y'^2 inside the fp16 range)
//   diag: S_k = 2^f_k (y'^2 . A_k + y' . B_k) + C_k
//   iso:  S_k = 2^f_k (y' . W_k + P_k |y|^2) + C_k
// with the fp16 panel (A, B, W) scaled per component by 2^-f_k so its
// entries stay in range; |y|^2 is fp32.  y' and y'^2 are rounded to fp16
// once, at staging; y'^2 above the fp16 maximum is clamped and reported.
// Statistics: [s1' | s2'] += gamma^T [y' | y'^2] on fp16 MFMA with gamma
// rounded to fp16; s0 (and the isotropic sum gamma |y|^2) in fp32 on the
// vector unit from the unrounded gamma.
//
// Work split: a workgroup owns a slice of 256 components, split over its
// waves (4 waves x 64 components, or 8 waves x 32 so that two waves share each
// SIMD within the register budget); each wave keeps its components' panel in
// registers.  32-point tiles are staged once per workgroup into LDS (row-
// major y' / y'^2 for the score operand, transposed copies for the statistics
// operand), double buffered, one barrier per tile plus one for the exchange
// of the waves' per-point (max, sum).  The slices of one point chunk are
// mapped to one XCD so X is read from HBM once and re-read from that L2.

#include <type_traits>

#include "largek_internal.h"

namespace gmm {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

constexpr int kT = kLkT;
constexpr float kLn2f = 0.69314718055994530942f;

template <int COV, int DP>
struct LkShape {
    static constexpr bool kIso = COV == GMM_COV_ISO;
    static constexpr int kNF = kIso ? 1 : 2;             // feature blocks: y' (, y'^2)
    static constexpr int kNPA = kIso ? 1 : 2;            // panel arrays: W (; A, B)
    static constexpr int kRowRM = DP + 8;                // halves per row-major row
    static constexpr int kRowT = kT + 4;                 // halves per transposed row
    static constexpr int kRM = kNF * kT * kRowRM;
    static constexpr int kTR = kNF * DP * kRowT;
    static constexpr int kBuf = kRM + kTR;               // halves per tile buffer
    static constexpr int kKS = DP / 32;                  // 32-dim MFMA steps
    static constexpr int kCB = DP / 8;                   // 8-column blocks per row
    static constexpr int kItems = (kT / 2) * kCB;        // staging items (row pair, col block)
};

__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
    const half2v h = {(_Float16)lo, (_Float16)hi};       // v_cvt_pk_f16_f32, round to nearest even
    return __builtin_bit_cast(uint32_t, h);
}

template <int N>
__device__ __forceinline__ float dpp_bcast(float v) {    // row_newbcast: lane N of each 16-lane row
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + N, 0xF, 0xF, false));
}

template <bool BF16>
__device__ __forceinline__ float h16_to_f32(uint32_t bits16) {
    if constexpr (BF16) return __uint_as_float(bits16 << 16);
    const uint16_t b = (uint16_t)bits16;
    return (float)__builtin_bit_cast(_Float16, b);
}

// Eight consecutive 16-bit elements of one row (zeros beyond column d on the
// element-wise path; the vector path needs d % 8 == 0 and col < d).
__device__ __forceinline__ uint4 load8(const uint16_t* __restrict__ row, int col, int d, bool vec) {
    if (vec) return *reinterpret_cast<const uint4*>(row + col);
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t lo = col + 2 * q < d ? row[col + 2 * q] : 0u;
        const uint32_t hi = col + 2 * q + 1 < d ? row[col + 2 * q + 1] : 0u;
        w[q] = lo | (hi << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

template <int COV, int DP, int MODE, bool BF16>
__global__ __launch_bounds__(64 * lk_waves(MODE, COV), lk_wg_per_cu(MODE)) void k_lk(const LkArgs a) {
    constexpr int WV = lk_waves(MODE, COV);          // waves per workgroup
    constexpr int KW = kLkSlice / WV;           // components per wave
    constexpr int KB = KW / 16;                 // 16-component blocks per wave
    constexpr int NT = 64 * WV;                 // threads per workgroup
    using Sh = LkShape<COV, DP>;
    constexpr bool kIso = Sh::kIso;
    constexpr int KS = Sh::kKS, NF = Sh::kNF;
    constexpr bool kStats = MODE == LK_FUSED_EM || MODE == LK_SWEEP2;
    constexpr bool kExchange = MODE != LK_SWEEP2;

    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * Sh::kBuf];
    __shared__ float2 dsc_l[DP];
    __shared__ __attribute__((aligned(16))) float nx2[2][kT];     // |y|^2 per point (isotropic)
    __shared__ __attribute__((aligned(16))) float lse_t[2][kT];   // merged base-2 LSE (sweep 2)
    __shared__ float2 wpart[WV][kT];   // per-wave (max, sum) of each point
    __shared__ int warg[WV][kT];
    __shared__ double llred[NT];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, j = lane & 15;
    const int G = gridDim.x, S = a.S;
    int slice, chunk;
    {
        const int b = blockIdx.x;
        if (G % (8 * S) == 0) {
            const int r = b >> 3;
            slice = r % S;
            chunk = (r / S) * 8 + (b & 7);
        } else {
            slice = b % S;
            chunk = b / S;
        }
    }
    const int nchunks = G / S;
    const int kbase = slice * kLkSlice + w * KW;
    const int64_t n = a.n;
    const int d = a.d;
    const bool want_arg = (MODE == LK_SWEEP1 && a.part_arg != nullptr) ||
                          (MODE == LK_FUSED_E && a.out_arg != nullptr);

    // ---- this wave's panel (registers), per-lane component constants
    half8 pw[Sh::kNPA][KS][KB];
#pragma unroll
    for (int pa = 0; pa < Sh::kNPA; ++pa)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                pw[pa][ks][kb] = __builtin_bit_cast(
                    half8, a.panel[((int64_t)(pa * KS + ks) * a.nblk + kbase / 16 + kb) * 64 + lane]);
    float cv[KB], fs[KB], pv[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const int k = kbase + 16 * kb + j;
        cv[kb] = a.cvec[k];   // -inf for padding components
        fs[kb] = a.fsc[k];
        pv[kb] = kIso ? a.pvec[k] : 0.0f;
    }
    for (int i = tid; i < DP; i += NT) dsc_l[i] = a.dsc[i];

    // ---- this chunk's tiles
    const int64_t tiles = (n + kT - 1) / kT;
    const int64_t tb = tiles / nchunks, tr = tiles % nchunks;
    const int64_t t0 = chunk * tb + (chunk < tr ? chunk : tr);
    const int64_t t1 = t0 + tb + (chunk < tr ? 1 : 0);

    f32x4 acc[kStats ? KB : 1][kStats ? NF : 1][kStats ? DP / 16 : 1];
    float s0acc[KB], s2acc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) s0acc[kb] = s2acc[kb] = 0.0f;
    if constexpr (kStats) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int f = 0; f < NF; ++f)
#pragma unroll
                for (int fc = 0; fc < DP / 16; ++fc) acc[kb][f][fc] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    double ll2 = 0.0;
    float sqmax = 0.0f;   // largest (y')^2 staged (diag): above the fp16 maximum it was clamped

    // ---- staging: item (row pair rp, 8-column block cb) per thread
    const bool item_on = tid < Sh::kItems;
    const int rp = tid / Sh::kCB, cb = tid % Sh::kCB;
    const int col0 = 8 * cb;
    const bool col_ok = col0 < d;
    const uint16_t* xb = reinterpret_cast<const uint16_t*>(a.x);
    uint4 raw0 = make_uint4(0, 0, 0, 0), raw1 = raw0;
    float lse_pf = 0.0f;
    int rows_in = 0;

    auto load_tile = [&](int64_t t) {
        const int64_t p0 = t * kT;
        const int64_t left = n - p0;
        rows_in = left >= kT ? kT : (int)left;
        if (item_on) {
            const int r0 = 2 * rp < rows_in ? 2 * rp : rows_in - 1;
            const int r1 = 2 * rp + 1 < rows_in ? 2 * rp + 1 : rows_in - 1;
            const int cc = col_ok ? col0 : 0;
            raw0 = load8(xb + (p0 + r0) * a.ldx, cc, d, a.vec);
            raw1 = load8(xb + (p0 + r1) * a.ldx, cc, d, a.vec);
        }
        if constexpr (MODE == LK_SWEEP2) {
            if (tid < kT) lse_pf = p0 + tid < n ? a.lse_in[p0 + tid] : INFINITY;   // gamma = 0
        }
    };

    auto store_tile = [&](int buf) {
        uint16_t* rm = lds + buf * Sh::kBuf;
        uint16_t* trp = rm + Sh::kRM;
        if (item_on) {
            uint32_t hy[2][4], hq[2][4];
            float yy[2];
            const uint4 rw[2] = {raw0, raw1};
            // rows beyond N and columns beyond D are zeroed only on ragged tiles
            auto stage_rows = [&](auto masked) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const bool row_ok = 2 * rp + h < rows_in;
                    const uint32_t wv[4] = {rw[h].x, rw[h].y, rw[h].z, rw[h].w};
                    float yp[8], ss = 0.0f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const uint32_t bits = (e & 1) ? (wv[e >> 1] >> 16) : (wv[e >> 1] & 0xFFFFu);
                        const float2 cs = dsc_l[col0 + e];
                        float y = h16_to_f32<BF16>(bits) - cs.x;
                        if constexpr (decltype(masked)::value) y = (row_ok && col0 + e < d) ? y : 0.0f;
                        if constexpr (kIso) ss = fmaf(y, y, ss);
                        yp[e] = y * cs.y;
                    }
                    yy[h] = ss;
#pragma unroll
                    for (int q = 0; q < 4; ++q) hy[h][q] = pack_h2(yp[2 * q], yp[2 * q + 1]);
                    if constexpr (!kIso) {
                        float y2[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float v = yp[e] * yp[e];
                            sqmax = fmaxf(sqmax, v);
                            y2[e] = fminf(v, kF16Max);
                        }
#pragma unroll
                        for (int q = 0; q < 4; ++q) hq[h][q] = pack_h2(y2[2 * q], y2[2 * q + 1]);
                    }
                }
            };
            if (rows_in == kT && d == DP) stage_rows(std::false_type{});
            else stage_rows(std::true_type{});
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int r = 2 * rp + h;
                *reinterpret_cast<uint4*>(rm + r * Sh::kRowRM + col0) =
                    make_uint4(hy[h][0], hy[h][1], hy[h][2], hy[h][3]);
                if constexpr (!kIso)
                    *reinterpret_cast<uint4*>(rm + (kT + r) * Sh::kRowRM + col0) =
                        make_uint4(hq[h][0], hq[h][1], hq[h][2], hq[h][3]);
            }
            if constexpr (kStats) {
                // transposed: feature row (col0 + e), points (2rp, 2rp + 1) as one dword
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int q = e >> 1;
                    const uint32_t v = (e & 1) ? ((hy[0][q] >> 16) | (hy[1][q] & 0xFFFF0000u))
                                               : ((hy[0][q] & 0xFFFFu) | (hy[1][q] << 16));
                    *reinterpret_cast<uint32_t*>(trp + (col0 + e) * Sh::kRowT + 2 * rp) = v;
                    if constexpr (!kIso) {
                        const uint32_t u = (e & 1) ? ((hq[0][q] >> 16) | (hq[1][q] & 0xFFFF0000u))
                                                   : ((hq[0][q] & 0xFFFFu) | (hq[1][q] << 16));
                        *reinterpret_cast<uint32_t*>(trp + (DP + col0 + e) * Sh::kRowT + 2 * rp) = u;
                    }
                }
            }
            if constexpr (kIso) {
                // |y|^2 of the two rows: the kCB lanes of a row pair are consecutive
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    float s = yy[h];
                    if constexpr (Sh::kCB >= 2) s += dpp<kDppXor1>(s);
                    if constexpr (Sh::kCB >= 4) s += dpp<kDppXor2>(s);
                    if constexpr (Sh::kCB >= 8) s += dpp<kDppHalfMirror>(s);
                    if constexpr (Sh::kCB >= 16) s += dpp<kDppMirror>(s);
                    yy[h] = s;
                }
                if (cb == 0) {
                    nx2[buf][2 * rp] = yy[0];
                    nx2[buf][2 * rp + 1] = yy[1];
                }
            }
        }
        if constexpr (MODE == LK_SWEEP2) {
            if (tid < kT) lse_t[buf][tid] = lse_pf;
        }
    };

    if (t0 < t1) {
        load_tile(t0);
        __syncthreads();   // dsc_l
        store_tile(0);
    }
    __syncthreads();

    for (int64_t t = t0; t < t1; ++t) {
        const int cur = (int)((t - t0) & 1);
        const uint16_t* rm = lds + cur * Sh::kBuf;
        const uint16_t* trp = rm + Sh::kRM;
        const int64_t prow = t * kT;
        if (t + 1 < t1) load_tile(t + 1);

        // ---- scores: 32 points x this wave's 64 components
        f32x4 sc[2][KB];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) sc[rb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        {
            // A operands (LDS) read two steps ahead of the MFMAs that use them;
            // step i = (pa, ks, rb); diag: y'^2 x A (pa 0), then y' x B (pa 1)
            constexpr int NA = Sh::kNPA * KS * 2;
            auto a_ptr = [&](int i) {
                const int pa = i / (2 * KS), ks = (i / 2) % KS, rb = i % 2;
                const int fb = kIso ? 0 : (pa == 0 ? 1 : 0);
                return reinterpret_cast<const uint4*>(rm + (fb * kT + 16 * rb + j) * Sh::kRowRM +
                                                      32 * ks + 8 * g);
            };
            uint4 a0 = *a_ptr(0), a1 = NA > 1 ? *a_ptr(1) : a0;
#pragma unroll
            for (int i = 0; i < NA; ++i) {
                const uint4 acur = a0;
                a0 = a1;
                if (i + 2 < NA) a1 = *a_ptr(i + 2);
                const int pa = i / (2 * KS), ks = (i / 2) % KS, rb = i % 2;
                const half8 av = __builtin_bit_cast(half8, acur);
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
                    sc[rb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pw[pa][ks][kb], sc[rb][kb], 0, 0, 0);
            }
        }
        float yyv[2][4];
        if constexpr (kIso) {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const float4 v = *reinterpret_cast<const float4*>(&nx2[cur][16 * rb + 4 * g]);
                yyv[rb][0] = v.x; yyv[rb][1] = v.y; yyv[rb][2] = v.z; yyv[rb][3] = v.w;
            }
        }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v = sc[rb][kb][r];
                    if constexpr (kIso) v = fmaf(pv[kb], yyv[rb][r], v);
                    sc[rb][kb][r] = fmaf(v, fs[kb], cv[kb]);
                }

        // ---- per point: base-2 LSE (and argmax) over the components
        float lse2[2][4];
        float lse_me = 0.0f;   // lanes j < 8: point 16 (j >> 2) + 4 g + (j & 3)
        int arg_me = 0;
        const int pt_me = 16 * (j >> 2) + 4 * g + (j & 3);
        float mw[2][4];   // this wave's per-point shift (fused E+M: reused for gamma)
        if constexpr (kExchange) {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float mx = sc[rb][0][r];
#pragma unroll
                    for (int kb = 1; kb < KB; ++kb) mx = fmaxf(mx, sc[rb][kb][r]);
                    const float m = row16_max(mx);
                    const float ms = m == -INFINITY ? 0.0f : m;
                    mw[rb][r] = ms;
                    float zz = 0.0f;
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) {
                        const float e = fast_exp2(sc[rb][kb][r] - ms);
                        if constexpr (kStats) sc[rb][kb][r] = e;   // exp(S - m_w), reused for gamma
                        zz += e;
                    }
                    const float z = row16_sum(zz);
                    if (j == 0) wpart[w][16 * rb + 4 * g + r] = make_float2(m, z);
                    if constexpr (!kStats) {
                        if (want_arg) {   // lowest component among this wave's maxima
                            int bi = 0x7FFFFFFF;
#pragma unroll
                            for (int kb = KB - 1; kb >= 0; --kb)
                                if (sc[rb][kb][r] == m) bi = kbase + 16 * kb + j;
                            const int arg = row16_min_i(bi);
                            if (j == 0) warg[w][16 * rb + 4 * g + r] = arg;
                        }
                    }
                }
            __syncthreads();
            if (j < 8) {
                float M = wpart[0][pt_me].x;
#pragma unroll
                for (int w2 = 1; w2 < WV; ++w2) M = fmaxf(M, wpart[w2][pt_me].x);
                const float Ms = M == -INFINITY ? 0.0f : M;
                float Z = 0.0f;
#pragma unroll
                for (int w2 = 0; w2 < WV; ++w2) {
                    const float2 mz = wpart[w2][pt_me];
                    Z = fmaf(mz.y, fast_exp2(mz.x - Ms), Z);
                }
                lse_me = Ms + fast_log2(Z);
                if (want_arg) {
                    arg_me = 0x7FFFFFFF;
#pragma unroll
                    for (int w2 = WV - 1; w2 >= 0; --w2)
                        if (wpart[w2][pt_me].x == M) arg_me = warg[w2][pt_me];
                }
            }
            const int64_t p = prow + pt_me;
            if constexpr (MODE == LK_SWEEP1) {
                if (w == 0 && j < 8 && p < n) {
                    a.part_lse[(int64_t)slice * n + p] = lse_me;
                    if (want_arg) {
                        float M = wpart[0][pt_me].x;
#pragma unroll
                        for (int w2 = 1; w2 < WV; ++w2) M = fmaxf(M, wpart[w2][pt_me].x);
                        a.part_arg[(int64_t)slice * n + p] = arg_me;
                        a.part_max[(int64_t)slice * n + p] = M;
                    }
                }
            } else {
                if (w == 0 && j < 8 && p < n) {
                    ll2 += (double)lse_me;
                    if constexpr (MODE == LK_FUSED_E) {
                        if (a.out_lse) a.out_lse[p] = lse_me * kLn2f;
                        if (want_arg) a.out_arg[p] = arg_me;
                    }
                }
                lse2[0][0] = dpp_bcast<0>(lse_me); lse2[0][1] = dpp_bcast<1>(lse_me);
                lse2[0][2] = dpp_bcast<2>(lse_me); lse2[0][3] = dpp_bcast<3>(lse_me);
                lse2[1][0] = dpp_bcast<4>(lse_me); lse2[1][1] = dpp_bcast<5>(lse_me);
                lse2[1][2] = dpp_bcast<6>(lse_me); lse2[1][3] = dpp_bcast<7>(lse_me);
            }
        } else {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const float4 v = *reinterpret_cast<const float4*>(&lse_t[cur][16 * rb + 4 * g]);
                lse2[rb][0] = v.x; lse2[rb][1] = v.y; lse2[rb][2] = v.z; lse2[rb][3] = v.w;
            }
        }
        (void)arg_me;

        // ---- responsibilities and statistics (registers -> MFMA)
        if constexpr (kStats) {
            if constexpr (MODE == LK_FUSED_EM) {
                // gamma = exp(S - m_w) * exp(m_w - lse); zero for rows beyond N
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const bool valid = prow + 16 * rb + 4 * g + r < n;
                        const float f = valid ? fast_exp2(mw[rb][r] - lse2[rb][r]) : 0.0f;
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb) sc[rb][kb][r] *= f;
                    }
            } else {
                // sweep 2: lse is +inf for rows beyond N, so gamma = 0 there
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb)
                            sc[rb][kb][r] = fast_exp2(sc[rb][kb][r] - lse2[rb][r]);
            }
            half8 ga[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                float s0 = 0.0f, s2 = 0.0f;
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        s0 += sc[rb][kb][r];
                        if constexpr (kIso) s2 = fmaf(sc[rb][kb][r], yyv[rb][r], s2);
                    }
                s0acc[kb] += s0;
                if constexpr (kIso) s2acc[kb] += s2;
                // gamma^T operand: component j, points 4g + e (e < 4) and 16 + 4g + e - 4
                ga[kb] = __builtin_bit_cast(
                    half8, make_uint4(pack_h2(sc[0][kb][0], sc[0][kb][1]), pack_h2(sc[0][kb][2], sc[0][kb][3]),
                                      pack_h2(sc[1][kb][0], sc[1][kb][1]), pack_h2(sc[1][kb][2], sc[1][kb][3])));
            }
            // B operands (transposed LDS rows) read one step ahead; step i = (f, fc)
            constexpr int NB = NF * (DP / 16);
            auto b_read = [&](int i) {
                const uint16_t* row = trp + (i * 16 + j) * Sh::kRowT;   // feature row f*DP + 16fc + j
                const uint2 b0 = *reinterpret_cast<const uint2*>(row + 4 * g);
                const uint2 b1 = *reinterpret_cast<const uint2*>(row + 16 + 4 * g);
                return make_uint4(b0.x, b0.y, b1.x, b1.y);
            };
            uint4 bnext = b_read(0);
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const half8 bv = __builtin_bit_cast(half8, bnext);
                if (i + 1 < NB) bnext = b_read(i + 1);
                const int f = i / (DP / 16), fc = i % (DP / 16);
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
                    acc[kb][f][fc] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ga[kb], bv, acc[kb][f][fc], 0, 0, 0);
            }
        }

        if (t + 1 < t1) store_tile(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: per-workgroup partials, one writer per value
    const int flag = __syncthreads_or(sqmax > kF16Max ? 1 : 0);
    if (tid == 0) a.part_flag[blockIdx.x] = flag;
    if constexpr (kStats) {
        const int ncol = kIso ? 2 + d : 1 + 2 * d;
        double* dst = a.part + (int64_t)blockIdx.x * kLkSlice * ncol;
        float* sred = reinterpret_cast<float*>(lds);   // [waves][4][KW][2]; the tiles are done
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            sred[((w * 4 + g) * KW + 16 * kb + j) * 2] = s0acc[kb];
            sred[((w * 4 + g) * KW + 16 * kb + j) * 2 + 1] = s2acc[kb];
        }
        __syncthreads();
        if (lane < KW) {
            const int kl = lane;   // one component per lane
            const float* s = sred + (w * 4 * KW + kl) * 2;
            const double s0 = ((double)s[0] + (double)s[2 * KW]) + ((double)s[4 * KW] + (double)s[6 * KW]);
            double* o = dst + (int64_t)(w * KW + kl) * ncol;
            o[0] = s0;
            if constexpr (kIso)
                o[1 + d] = ((double)s[1] + (double)s[2 * KW + 1]) + ((double)s[4 * KW + 1] + (double)s[6 * KW + 1]);
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int f = 0; f < NF; ++f)
#pragma unroll
                for (int fc = 0; fc < DP / 16; ++fc) {
                    const int dd = 16 * fc + j;
                    if (dd < d) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int kl = w * KW + 16 * kb + 4 * g + r;
                            dst[(int64_t)kl * ncol + 1 + f * d + dd] = (double)acc[kb][f][fc][r];
                        }
                    }
                }
    }
    if constexpr (MODE == LK_FUSED_EM || MODE == LK_FUSED_E) {
        llred[tid] = ll2;
        __syncthreads();
        for (int s2 = NT / 2; s2 > 0; s2 >>= 1) {
            if (tid < s2) llred[tid] += llred[tid + s2];
            __syncthreads();
        }
        if (tid == 0) a.part_ll[blockIdx.x] = llred[0] * kLn2;
    }
}

template <int COV, int DP, int MODE>
hipError_t launch3(const Plan& p, const LkArgs& a, int grid, hipStream_t s) {
    if (p.xdt == GMM_BF16)
        hipLaunchKernelGGL((k_lk<COV, DP, MODE, true>), dim3(grid), dim3(64 * lk_waves(MODE, COV)), 0, s, a);
    else
        hipLaunchKernelGGL((k_lk<COV, DP, MODE, false>), dim3(grid), dim3(64 * lk_waves(MODE, COV)), 0, s, a);
    return hipGetLastError();
}

template <int COV, int MODE>
hipError_t launch2(const Plan& p, const LkArgs& a, int grid, hipStream_t s) {
    switch (p.dp) {
        case 32: return launch3<COV, 32, MODE>(p, a, grid, s);
        case 64: return launch3<COV, 64, MODE>(p, a, grid, s);
        case 128: return launch3<COV, 128, MODE>(p, a, grid, s);
    }
    return hipErrorInvalidValue;
}

template <int COV>
hipError_t launch1(const Plan& p, const LkArgs& a, int mode, int grid, hipStream_t s) {
    switch (mode) {
        case LK_FUSED_EM: return launch2<COV, LK_FUSED_EM>(p, a, grid, s);
        case LK_SWEEP1: return launch2<COV, LK_SWEEP1>(p, a, grid, s);
        case LK_SWEEP2: return launch2<COV, LK_SWEEP2>(p, a, grid, s);
        case LK_FUSED_E: return launch2<COV, LK_FUSED_E>(p, a, grid, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t lk_launch(const Plan& p, const LkArgs& a, int mode, int grid, hipStream_t s) {
    if (p.cov == GMM_COV_ISO) return launch1<GMM_COV_ISO>(p, a, mode, grid, s);
    return launch1<GMM_COV_DIAG>(p, a, mode, grid, s);
}

}  // namespace gmm
