// Fused E-step + M-step statistics for a diagonal-covariance GMM, fp32 math.
//
// Method: [Flash-GMM] Method, fused E-M step (tile X along N; per tile the
// Mahalanobis terms and the softmax over all K stay on chip; s0/s1/s2 are
// accumulated in the same pass, the N x K responsibilities never reach HBM).
// Density and posterior: [LP-GMM] 1.1-1.2; log-space posterior with max
// shift: [LP-GMM] 4.2; exp, log, denominators and statistics in fp32 or wider
// whatever the storage type: [LP-GMM] 1.3, 2.1.
//
// Score as a contraction.  For a diagonal covariance
//   log2(pi_k N(x | mu_k, sigma_k^2)) = sum_d a_kd x_d^2 + b_kd x_d + c_k,
//   a_kd = -1/2 log2(e) / sigma_kd^2,  b_kd = log2(e) mu_kd / sigma_kd^2,
//   c_k  = log2(e) (log pi_k - 1/2 (D log 2pi + sum_d log sigma_kd^2
//                                   + sum_d mu_kd^2 / sigma_kd^2)),
// so a 16-point x 16-component score block is [x^2 | x] (16 x 2D) times the
// panel [a ; b] (2D x 16): v_mfma_f32_16x16x4f32 steps with the accumulator
// initialised to c_k.  The accumulator layout of that product (lane (g, j)
// holds points 4g+r of component j) is exactly the A-operand layout of
// gamma^T in the statistics product [S1 | S2] += gamma^T [x | x^2], so gamma
// goes from the exp straight into the next MFMAs without leaving registers.
// The log-sum-exp over the 16 components of a block is a 4-step DPP
// butterfly inside each 16-lane row.
//
// Centring: X is shifted by the fixed per-dimension centre c (mean of the
// heaviest prepared component) on its way into LDS, the panel is built from
// mu - c, and S1 / S2 are moments about c.  The expanded quadratic then
// cancels only at the scale of the data's spread, not of its offset.
//
// Work split: a workgroup of W waves owns a contiguous range of 16*W-point
// tiles; each wave computes one 16-point group per tile.  Tiles are staged
// global -> registers -> LDS with coalesced 16-byte loads, converted to fp32
// (block conversion, [LP-GMM] 3.3) and double buffered, so the loads of
// tile t+1 are in flight while tile t is computed.  Each workgroup writes
// one fp64 partial of (s0, S1, S2) and of LL; later kernels sum them in a
// fixed order (no cross-workgroup synchronisation here: an agent-scope
// fence per workgroup would write back and invalidate the whole L2 of its
// XCD while the others are still streaming X).
//
// This translation unit is compiled with IEEE mode off and no-NaN
// assumptions so that the DPP max folds into one v_max_f32_dpp per step;
// nothing here tests floats for NaN (non-finite results are detected by the
// kernels that consume the partials).

#include "diag_internal.h"

namespace gmm {

namespace {

template <int DP, int KB, int WAVES>
struct FusedShape {
    static constexpr int kThreads = 64 * WAVES;
    static constexpr int kRow = DP + 4;                    // LDS row stride (floats)
    static constexpr int kSlot = 16 * kRow;                // one 16-point group
    static constexpr int kWaveLds = 3 * kSlot;             // per-wave ring of 3 groups
    static constexpr int kXFloats = WAVES * kWaveLds;
    static constexpr int kRedFloats = WAVES * 16 * KB * 2 * DP;
    static constexpr int kSmem = kXFloats > kRedFloats ? kXFloats : kRedFloats;
};

// Global -> registers -> LDS staging of one 16-point group by one wave.
// Loads always read a clamped in-bounds address; rows beyond N and columns
// beyond D are zeroed only when the group is staged into LDS.  (Masking the
// register right after the load would make the compiler wait for the load
// to land, which would serialise the prefetch.)  The vector path keeps each
// lane on fixed columns (its centre values stay in registers); the
// element-wise path reads the centre from LDS.
template <typename XT, int DP, bool VEC>
struct GroupLoader {
    static constexpr int kEV = VEC ? Vec16<XT>::kElems : 1;
    static constexpr int kVPR = DP / kEV;                  // vectors (elements) per row
    static constexpr int kNV = 16 * kVPR;                  // per group
    static constexpr int kPer = (kNV + 63) / 64;
    static constexpr int kRow = DP + 4;
    static_assert(!VEC || 64 % kVPR == 0, "vector geometry");

    uint4 raw[VEC ? kPer : 1];
    float sc[VEC ? 1 : kPer];
    float sh[VEC ? kEV : 1];
    int lane;
    int rows;        // rows of the loaded group that exist (uniform)
    bool colok;      // this lane's columns are inside D (vector path)

    __device__ __forceinline__ void init(int ln, int d, const float* __restrict__ shift) {
        lane = ln;
        rows = 0;
        if constexpr (VEC) {
            const int col = (lane % kVPR) * kEV;
            colok = col < d;
#pragma unroll
            for (int e = 0; e < kEV; ++e) sh[e] = shift[col + e];
        } else {
            colok = true;
            sh[0] = 0.0f;
        }
    }

    // gq: global group index (must be a valid group: gq * 16 < n).
    __device__ __forceinline__ void load(const XT* __restrict__ x, int64_t n, int d, int64_t ldx,
                                         int64_t gq) {
        const int64_t p0 = gq * 16;
        const XT* __restrict__ gb = x + p0 * ldx;
        const int64_t left = n - p0;
        rows = left >= 16 ? 16 : (int)left;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int v = lane + 64 * i;
            const int r = v / kVPR;
            const int col = (v % kVPR) * kEV;
            const int rc = r < rows ? r : rows - 1;
            if constexpr (VEC) {
                const uint32_t off = (uint32_t)rc * (uint32_t)ldx + (uint32_t)(colok ? col : 0);
                raw[i] = *reinterpret_cast<const uint4*>(gb + off);
            } else {
                const uint32_t off = (uint32_t)rc * (uint32_t)ldx + (uint32_t)(col < d ? col : 0);
                sc[i] = to_f32(gb[off]);
            }
        }
    }

    __device__ __forceinline__ void store(float* __restrict__ slot, int d,
                                          const float* __restrict__ shift_lds) const {
        const bool full = rows == 16 && d == DP;   // uniform: no masking needed
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int v = lane + 64 * i;
            if (kNV % 64 != 0 && v >= kNV) continue;
            const int r = v / kVPR;
            const int col = (v % kVPR) * kEV;
            if constexpr (VEC) {
                float tmp[kEV];
                Vec16<XT>::unpack(raw[i], tmp);
                const bool ok = full || (colok && r < rows);
                float4* dst = reinterpret_cast<float4*>(slot + r * kRow + col);
#pragma unroll
                for (int e = 0; e < kEV / 4; ++e)
                    dst[e] = ok ? make_float4(tmp[4 * e] - sh[4 * e], tmp[4 * e + 1] - sh[4 * e + 1],
                                              tmp[4 * e + 2] - sh[4 * e + 2], tmp[4 * e + 3] - sh[4 * e + 3])
                                : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            } else {
                const bool ok = r < rows && col < d;
                slot[r * kRow + col] = ok ? sc[i] - shift_lds[col] : 0.0f;
            }
        }
    }
};

template <int N>
__device__ __forceinline__ void lds_load(const float* __restrict__ p, float* o) {
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            const float4 v = reinterpret_cast<const float4*>(p)[i];
            o[4 * i] = v.x; o[4 * i + 1] = v.y; o[4 * i + 2] = v.z; o[4 * i + 3] = v.w;
        }
    } else if constexpr (N == 2) {
        const float2 v = *reinterpret_cast<const float2*>(p);
        o[0] = v.x; o[1] = v.y;
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) o[i] = p[i];
    }
}

__device__ __forceinline__ bool f64_nonfinite(double v) {
    const unsigned long long b = (unsigned long long)__double_as_longlong(v);
    return ((b >> 52) & 0x7ffull) == 0x7ffull;
}

// Order this wave's LDS writes before its later LDS reads (one wave: no
// s_barrier needed, only a compiler/memory fence at wavefront scope).
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Scores of one 16-point group: accumulators seeded with c_k, then
// [x^2 | x] . [a ; b].  Lane (g, j) supplies point j, dims g*DP/4 ...
template <int DP, int KB>
__device__ __forceinline__ void group_scores(const float* __restrict__ slot, int g, int j,
                                             const float (&wa)[DP / 4][KB],
                                             const float (&wb)[DP / 4][KB], const float (&cv)[KB],
                                             f32x4 (&sc)[KB]) {
    constexpr int kRow = DP + 4;
#pragma unroll
    for (int b = 0; b < KB; ++b) sc[b] = f32x4{cv[b], cv[b], cv[b], cv[b]};
    const float* xr = slot + j * kRow + g * (DP / 4);
#pragma unroll
    for (int s0 = 0; s0 < DP / 4; s0 += 4) {
        const float4 xv = *reinterpret_cast<const float4*>(xr + s0);
        const float xq[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float x1 = xq[q], x2 = x1 * x1;
#pragma unroll
            for (int b = 0; b < KB; ++b) {
                sc[b] = mfma16x16x4(x2, wa[s0 + q][b], sc[b]);
                sc[b] = mfma16x16x4(x1, wb[s0 + q][b], sc[b]);
            }
        }
    }
}

// One pipeline step for group q of this wave: (a) scores of group q+1 next
// to (b) the log-sum-exp of group q, (c) statistics of group q, (d) staging
// of group q+2 from `ld` into the free ring slot and the global loads of
// group q+4 into `ld` (two register sets alternate, so the loads of a group
// are issued two steps before its staging).
template <int DP, int KB, typename XT, bool VEC, bool EM>
struct Step {
    static constexpr int kRow = DP + 4, kSlot = 16 * kRow;

    __device__ __forceinline__ static void run(
        int q, int ng, int64_t q0, int64_t qlast, int64_t n, int d, int64_t ldx, int k_real,
        int g, int j, const XT* __restrict__ x, float* ring, int& s_cur, int& s_nxt, int& s_new,
        GroupLoader<XT, DP, VEC>& ld, const float* __restrict__ shift_lds,
        const float (&wa)[DP / 4][KB], const float (&wb)[DP / 4][KB], const float (&cv)[KB],
        f32x4 (&sc)[KB], f32x4 (&acc1)[KB][DP / 16], f32x4 (&acc2)[KB][DP / 16],
        float (&s0acc)[KB], double& ll2, float* __restrict__ out_lse, int* __restrict__ out_arg) {
        // (a)
        f32x4 sn[KB];
        group_scores<DP, KB>(ring + s_nxt * kSlot, g, j, wa, wb, cv, sn);

        // (b) base-2 log-sum-exp (lane: points 4g+r of component 16b+j)
        float m[4], z[4], e[KB][4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float mx = sc[0][r];
#pragma unroll
            for (int b = 1; b < KB; ++b) mx = fmaxf(mx, sc[b][r]);
            m[r] = row16_max(mx);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float zz = 0.0f;
#pragma unroll
            for (int b = 0; b < KB; ++b) {
                e[b][r] = fast_exp2(sc[b][r] - m[r]);
                zz += e[b][r];
            }
            z[r] = row16_sum(zz);
        }
        // rows of this group that exist (0 for a padding step past the run)
        const int64_t left = q < ng ? n - (q0 + q) * 16 : 0;
        const int rows = left >= 16 ? 16 : (int)left;
        float lse2[4];
        bool valid[4];
        float tll = 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            lse2[r] = m[r] + fast_log2(z[r]);
            valid[r] = 4 * g + r < rows;
            tll += valid[r] ? lse2[r] : 0.0f;
        }
        ll2 += (double)tll;

        const float* xs = ring + s_cur * kSlot;
        if constexpr (EM) {
            // (c) gamma stays in registers: s0, [S1 | S2] += gamma^T [x | x^2]
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float inv = valid[r] ? __builtin_amdgcn_rcpf(z[r]) : 0.0f;
#pragma unroll
                for (int b = 0; b < KB; ++b) e[b][r] *= inv;
            }
#pragma unroll
            for (int b = 0; b < KB; ++b) s0acc[b] += (e[b][0] + e[b][1]) + (e[b][2] + e[b][3]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float xv[DP / 16];
                lds_load<DP / 16>(xs + (4 * g + r) * kRow + j * (DP / 16), xv);
#pragma unroll
                for (int c = 0; c < DP / 16; ++c) {
                    const float x1 = xv[c], x2 = x1 * x1;
#pragma unroll
                    for (int b = 0; b < KB; ++b) {
                        acc1[b][c] = mfma16x16x4(e[b][r], x1, acc1[b][c]);
                        acc2[b][c] = mfma16x16x4(e[b][r], x2, acc2[b][c]);
                    }
                }
            }
        } else {
            const int64_t pbase = (q0 + q) * 16 + 4 * g;
            if (out_lse != nullptr && j == 0) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (valid[r]) out_lse[pbase + r] = (float)((double)lse2[r] * kLn2);
            }
            if (out_arg != nullptr) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    int best = 0x7fffffff;
#pragma unroll
                    for (int b = KB - 1; b >= 0; --b)
                        if (sc[b][r] == m[r] && 16 * b + j < k_real) best = 16 * b + j;
                    best = row16_min_i(best);
                    if (j == 0 && valid[r]) out_arg[pbase + r] = best;
                }
            }
        }

        // (d)
        ld.store(ring + s_new * kSlot, d, shift_lds);
        const int64_t qn = q0 + q + 4;
        ld.load(x, n, d, ldx, qn <= qlast ? qn : qlast);
        wave_lds_fence();
#pragma unroll
        for (int b = 0; b < KB; ++b) sc[b] = sn[b];
        const int t = s_cur;
        s_cur = s_nxt;
        s_nxt = s_new;
        s_new = t;
    }
};

// EM = true: E-step + statistics + LL; EM = false: E-step only (loglik).
//
// Each wave owns a contiguous run of 16-point groups and pipelines them
// through a private 3-slot LDS ring, with the global loads of a group issued
// two steps before it is staged (two register sets).  In step q the score
// MFMAs of group q+1 sit next to the log-sum-exp of group q, the statistics
// MFMAs of group q next to the staging of group q+2.  No workgroup barrier
// is taken inside the loop.
template <int DP, int KB, typename XT, bool VEC, bool EM, int WAVES, int OCC>
__global__ __launch_bounds__(64 * WAVES, OCC) void k_diag_fused(
    const XT* __restrict__ x, int64_t n, int d, int64_t ldx, int k_real,
    const float* __restrict__ panel, const float* __restrict__ th_pi,
    const double* __restrict__ chunk_part, int nch, const float* __restrict__ shift,
    double* __restrict__ part, double* __restrict__ part_ll,
    float* __restrict__ out_lse, int* __restrict__ out_arg) {
    using S = FusedShape<DP, KB, WAVES>;
    using St = Step<DP, KB, XT, VEC, EM>;
    constexpr int THREADS = S::kThreads;
    __shared__ __attribute__((aligned(16))) float smem[S::kSmem];
    __shared__ float s0red[WAVES][4][16 * KB];
    __shared__ float shift_lds[DP];
    __shared__ double llred[THREADS];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6, g = lane >> 4, j = lane & 15;

    // Score panel and per-component constants stay in registers.
    float wa[DP / 4][KB], wb[DP / 4][KB], cv[KB];
#pragma unroll
    for (int s = 0; s < DP / 4; ++s)
#pragma unroll
        for (int b = 0; b < KB; ++b) {
            wa[s][b] = panel[((s * 2) * KB + b) * 64 + lane];
            wb[s][b] = panel[((s * 2 + 1) * KB + b) * 64 + lane];
        }
    // log2-normaliser of component 16b+j from the prepared per-chunk sums:
    // c_k = log2(e) (log pi_k - 1/2 (D log 2pi + sum log var + sum (mu-c)^2/var))
#pragma unroll
    for (int b = 0; b < KB; ++b) {
        const int k = 16 * b + j;
        if (k < k_real) {
            double sl = 0.0, sm = 0.0;
            for (int ch = 0; ch < nch; ++ch) {
                sl += chunk_part[((int64_t)k * nch + ch) * 4 + 0];
                sm += chunk_part[((int64_t)k * nch + ch) * 4 + 1];
            }
            cv[b] = (float)((log((double)th_pi[k]) - 0.5 * (d * kLog2Pi + sl + sm)) * kLog2e);
        } else {
            cv[b] = -INFINITY;   // padding component: weight 0
        }
    }
    for (int dd = tid; dd < DP; dd += THREADS) shift_lds[dd] = shift[dd];
    __syncthreads();

    // this wave's run of groups
    const int64_t groups = (n + 15) / 16;
    const int64_t nw = (int64_t)gridDim.x * WAVES, gw = (int64_t)blockIdx.x * WAVES + w;
    const int64_t gbase = groups / nw, grem = groups % nw;
    const int64_t q0 = gw * gbase + (gw < grem ? gw : grem);
    const int ng = (int)(gbase + (gw < grem ? 1 : 0));
    const int64_t qlast = q0 + ng - 1;

    f32x4 acc1[KB][DP / 16], acc2[KB][DP / 16];
    float s0acc[KB];
#pragma unroll
    for (int b = 0; b < KB; ++b) {
        s0acc[b] = 0.0f;
#pragma unroll
        for (int c = 0; c < DP / 16; ++c) {
            acc1[b][c] = f32x4{0.f, 0.f, 0.f, 0.f};
            acc2[b][c] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    double ll2 = 0.0;

    float* ring = smem + w * S::kWaveLds;
    if (ng > 0) {
        GroupLoader<XT, DP, VEC> la, lb;
        la.init(lane, d, shift);
        lb.init(lane, d, shift);
        auto clampq = [&](int64_t qq) { return qq <= qlast ? qq : qlast; };
        // prologue: groups 0, 1 staged, group 0 scored, groups 2, 3 in flight
        la.load(x, n, d, ldx, q0);
        lb.load(x, n, d, ldx, clampq(q0 + 1));
        la.store(ring, d, shift_lds);
        lb.store(ring + S::kSlot, d, shift_lds);
        la.load(x, n, d, ldx, clampq(q0 + 2));
        lb.load(x, n, d, ldx, clampq(q0 + 3));
        wave_lds_fence();
        f32x4 sc[KB];
        group_scores<DP, KB>(ring, g, j, wa, wb, cv, sc);
        int s_cur = 0, s_nxt = 1, s_new = 2;
        for (int q = 0; q < ng; q += 2) {
            St::run(q, ng, q0, qlast, n, d, ldx, k_real, g, j, x, ring, s_cur, s_nxt, s_new, la,
                    shift_lds, wa, wb, cv, sc, acc1, acc2, s0acc, ll2, out_lse, out_arg);
            St::run(q + 1, ng, q0, qlast, n, d, ldx, k_real, g, j, x, ring, s_cur, s_nxt, s_new, lb,
                    shift_lds, wa, wb, cv, sc, acc1, acc2, s0acc, ll2, out_lse, out_arg);
        }
    }

    // ---- one fp64 partial per workgroup, waves summed in a fixed order
    __syncthreads();   // every wave is done with its ring before the LDS is reused
    llred[tid] = (j == 0) ? ll2 : 0.0;
    if constexpr (EM) {
        float* red = smem;
#pragma unroll
        for (int b = 0; b < KB; ++b)
#pragma unroll
            for (int c = 0; c < DP / 16; ++c)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int comp = 16 * b + 4 * g + q;
                    float* row = red + (w * 16 * KB + comp) * (2 * DP);
                    row[j * (DP / 16) + c] = acc1[b][c][q];
                    row[DP + j * (DP / 16) + c] = acc2[b][c][q];
                }
#pragma unroll
        for (int b = 0; b < KB; ++b) s0red[w][g][16 * b + j] = s0acc[b];
    }
    __syncthreads();
    const int64_t wg = blockIdx.x, G = gridDim.x;
    if constexpr (EM) {
        // partial columns: [s0, S1_0, S2_0, S1_1, S2_1, ...] (moments about c)
        const int ncol = 1 + 2 * d;
        const float* red = smem;
        for (int e2 = tid; e2 < k_real * ncol; e2 += THREADS) {
            const int k = e2 / ncol, c = e2 % ncol;
            double v = 0.0;
            if (c == 0) {
                for (int w2 = 0; w2 < WAVES; ++w2)
                    for (int g2 = 0; g2 < 4; ++g2) v += (double)s0red[w2][g2][k];
            } else {
                const int dd = (c - 1) >> 1, mom = (c - 1) & 1;
                const int col = mom * DP + dd;
                for (int w2 = 0; w2 < WAVES; ++w2)
                    v += (double)red[(w2 * 16 * KB + k) * (2 * DP) + col];
            }
            part[(wg * k_real + k) * ncol + c] = v;
        }
    }
    if (tid == 0) {
        double s = 0.0;
        for (int i = 0; i < THREADS; ++i) s += llred[i];
        part_ll[wg] = s * kLn2;
    }

}

template <int DP, int KB, typename XT, bool VEC, bool EM>
hipError_t launch_t(const Plan& p, const DiagWs& w, const void* x, int grid, float* lse,
                    int* arg, hipStream_t s) {
    constexpr int W = diag_waves(DP);
    hipLaunchKernelGGL((k_diag_fused<DP, KB, XT, VEC, EM, W, kDiagWgPerCu>), dim3(grid),
                       dim3(64 * W), 0, s, (const XT*)x, p.n, (int)p.d, p.ldx, (int)p.k,
                       w.panel, w.pi, w.chunk_part, diag_chunks(p), w.shift, w.part, w.part_ll,
                       lse, arg);
    return hipGetLastError();
}

template <int DP, int KB, bool EM>
hipError_t launch_x(const Plan& p, const DiagWs& w, const void* x, bool vec, int grid,
                    float* lse, int* arg, hipStream_t s) {
    switch (p.xdt) {
        case GMM_F32:
            return vec ? launch_t<DP, KB, float, true, EM>(p, w, x, grid, lse, arg, s)
                       : launch_t<DP, KB, float, false, EM>(p, w, x, grid, lse, arg, s);
        case GMM_BF16:
            return vec ? launch_t<DP, KB, bf16_t, true, EM>(p, w, x, grid, lse, arg, s)
                       : launch_t<DP, KB, bf16_t, false, EM>(p, w, x, grid, lse, arg, s);
        default:
            return vec ? launch_t<DP, KB, _Float16, true, EM>(p, w, x, grid, lse, arg, s)
                       : launch_t<DP, KB, _Float16, false, EM>(p, w, x, grid, lse, arg, s);
    }
}

bool x_vec_ok(const Plan& p, const void* x) {
    const int es = p.xdt == GMM_F32 ? 4 : 2;
    const int ev = 16 / es;
    return ((uintptr_t)x % 16 == 0) && ((p.ldx * es) % 16 == 0) && (p.d % ev == 0);
}

}  // namespace

hipError_t diag_launch_fused(const Plan& p, const DiagWs& w, const void* x, bool em, int grid,
                             float* lse, int* arg, hipStream_t s) {
    const bool vec = x_vec_ok(p, x);
#define CASE(DP_, KB_)                                                                          \
    if (p.dp == DP_ && p.kb == KB_)                                                             \
        return em ? launch_x<DP_, KB_, true>(p, w, x, vec, grid, lse, arg, s)                  \
                  : launch_x<DP_, KB_, false>(p, w, x, vec, grid, lse, arg, s);
    GMM_DIAG_SHAPES(CASE)
#undef CASE
    return hipErrorInvalidValue;
}

}  // namespace gmm
