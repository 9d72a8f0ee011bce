// Diagonal-covariance GMM EM iteration with fp32 math, K <= 64, D <= 128.
//
// Method: [Flash-GMM] Method, fused E-M step (tile X along N; per tile the
// Mahalanobis terms and the softmax over all K stay on chip; s0/s1/s2 are
// accumulated in the same pass).  Density and posterior: [LP-GMM] 1.1-1.2;
// log-space posterior with max shift: [LP-GMM] 4.2; precision rules (exp,
// log, denominators and statistics in fp32 or wider): [LP-GMM] 1.3, 2.1.
//
// Score as a contraction.  For a diagonal covariance
//   log2(pi_k N(x | mu_k, sigma_k^2)) = sum_d a_kd x_d^2 + b_kd x_d + c_k,
//   a_kd = -1/2 log2(e) / sigma_kd^2,  b_kd = log2(e) mu_kd / sigma_kd^2,
//   c_k  = log2(e) (log pi_k - 1/2 (D log 2pi + sum_d log sigma_kd^2
//                                   + sum_d mu_kd^2 / sigma_kd^2)),
// so a 16-point x 16-component score block is [x^2 | x] (16 x 2D) times the
// panel [a ; b] (2D x 16): v_mfma_f32_16x16x4f32 steps.  The accumulator
// layout of that product (lane (g, j) holds points 4g+r of component j) is
// exactly the A-operand layout of gamma^T in the statistics product
// [s1 | s2] += gamma^T [x | x^2], so gamma never leaves registers.
//
// Centring.  The expanded form cancels when |x| is large against sigma, so
// X is shifted by a fixed per-dimension centre c (the mean of the heaviest
// component of the parameters given to gmm_prepare) on its way into
// LDS, the panel is built from mu - c, and the statistics are accumulated
// about c: S1 = sum gamma (x - c), S2 = sum gamma (x - c)^2.  Finalize turns
// them back into raw moments in fp64.
//
// Work split: one workgroup = 4 waves = 64-point tiles, a contiguous range of
// tiles per workgroup, X double-buffered through LDS with coalesced 16-byte
// loads (converted to fp32 on the way, [LP-GMM] 3.3 block conversion).
// Each workgroup writes one fp64 partial of (s0, S1, S2, LL); the
// reduce-finalize kernel sums the partials in a fixed order (deterministic),
// computes the M-step and prepares the panel for the next iteration.

#include "common.h"
#include "plan.h"

namespace gmm {

namespace {

constexpr int kTile = 64;
constexpr int kThreads = 256;

template <int DP, int KB>
struct Shape {
    static constexpr int kRow = DP + 4;                    // LDS row stride, floats
    static constexpr int kXFloats = 2 * kTile * kRow;      // two tile buffers
    static constexpr int kRedFloats = 4 * 16 * KB * 2 * DP;
    static constexpr int kSmem = kXFloats > kRedFloats ? kXFloats : kRedFloats;
    static constexpr int kPanel = (DP / 4) * 2 * KB * 64;
};

// Global -> registers -> LDS staging of one 64-point tile.
template <typename XT, int DP, bool VEC>
struct TileLoader {
    static constexpr int kEV = VEC ? Vec16<XT>::kElems : 1;
    static constexpr int kNV = kTile * DP / kEV;
    static constexpr int kPer = (kNV + kThreads - 1) / kThreads;
    static constexpr int kRow = DP + 4;
    uint4 raw[VEC ? kPer : 1];
    float sc[VEC ? 1 : kPer];
    float sh[kEV];   // centre of the columns this thread stages (fixed per thread)

    __device__ __forceinline__ void load_shift(const float* __restrict__ shift) {
        const int col = VEC ? (threadIdx.x % (DP / kEV)) * kEV : threadIdx.x % DP;
#pragma unroll
        for (int e = 0; e < kEV; ++e) sh[e] = shift[col + e];
    }

    __device__ __forceinline__ void load(const XT* __restrict__ x, int64_t n, int d, int64_t ldx,
                                         int64_t tile) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int v = threadIdx.x + i * kThreads;
            if constexpr (VEC) {
                const int row = v / (DP / kEV);
                const int col = (v % (DP / kEV)) * kEV;
                const int64_t p = tile * kTile + row;
                if (v < kNV && p < n && col < d)
                    raw[i] = *reinterpret_cast<const uint4*>(x + p * ldx + col);
                else
                    raw[i] = make_uint4(0, 0, 0, 0);
            } else {
                const int row = v / DP;
                const int col = v % DP;
                const int64_t p = tile * kTile + row;
                sc[i] = (v < kNV && p < n && col < d) ? to_f32(x[p * ldx + col]) : 0.0f;
            }
        }
    }

    __device__ __forceinline__ void store(float* __restrict__ buf) const {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int v = threadIdx.x + i * kThreads;
            if (v >= kNV) continue;
            if constexpr (VEC) {
                const int row = v / (DP / kEV);
                const int col = (v % (DP / kEV)) * kEV;
                float tmp[kEV];
                Vec16<XT>::unpack(raw[i], tmp);
#pragma unroll
                for (int e = 0; e < kEV; ++e) tmp[e] -= sh[e];
                float4* dst = reinterpret_cast<float4*>(buf + row * kRow + col);
#pragma unroll
                for (int e = 0; e < kEV / 4; ++e)
                    dst[e] = make_float4(tmp[4 * e], tmp[4 * e + 1], tmp[4 * e + 2], tmp[4 * e + 3]);
            } else {
                const int row = v / DP;
                const int col = v % DP;
                buf[row * kRow + col] = sc[i] - sh[0];
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

// EM = true: E-step + statistics; EM = false: E-step only (loglik).
template <int DP, int KB, typename XT, bool VEC, bool EM>
__global__ __launch_bounds__(kThreads, 2) void k_diag_fused(
    const XT* __restrict__ x, int64_t n, int d, int64_t ldx, int k_real,
    const float* __restrict__ panel, const float* __restrict__ cvec,
    const float* __restrict__ shift, int64_t tiles,
    double* __restrict__ part, double* __restrict__ part_ll,
    float* __restrict__ out_lse, int* __restrict__ out_arg,
    double* __restrict__ ll_ws, double* __restrict__ ll_out, int* __restrict__ nonfinite_ll,
    unsigned int* __restrict__ arrivals) {
    using S = Shape<DP, KB>;
    __shared__ __attribute__((aligned(16))) float smem[S::kSmem];
    __shared__ float s0red[4][4][16 * KB];
    __shared__ double llred[kThreads];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6, g = lane >> 4, j = lane & 15;

    // Score panel and constants live in registers for the whole kernel.
    float wa[DP / 4][KB], wb[DP / 4][KB], cv[KB];
#pragma unroll
    for (int s = 0; s < DP / 4; ++s)
#pragma unroll
        for (int b = 0; b < KB; ++b) {
            wa[s][b] = panel[((s * 2) * KB + b) * 64 + lane];
            wb[s][b] = panel[((s * 2 + 1) * KB + b) * 64 + lane];
        }
#pragma unroll
    for (int b = 0; b < KB; ++b) cv[b] = cvec[16 * b + j];

    const int64_t G = gridDim.x, wg = blockIdx.x;
    const int64_t base = tiles / G, rem = tiles % G;
    const int64_t t0 = wg * base + (wg < rem ? wg : rem);
    const int64_t t1 = t0 + base + (wg < rem ? 1 : 0);

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

    TileLoader<XT, DP, VEC> ld;
    ld.load_shift(shift);
    if (t0 < t1) {
        ld.load(x, n, d, ldx, t0);
        ld.store(smem);
    }
    __syncthreads();

    for (int64_t t = t0; t < t1; ++t) {
        const int cur = (int)((t - t0) & 1);
        const float* xs = smem + cur * kTile * S::kRow;
        if (t + 1 < t1) ld.load(x, n, d, ldx, t + 1);

        // ---- scores: [x^2 | x] . [a ; b]  (lane (g, j): point w*16+j, dims g*DP/4 ..)
        f32x4 sc[KB];
#pragma unroll
        for (int b = 0; b < KB; ++b) sc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
        const float* xr = xs + (w * 16 + j) * S::kRow + g * (DP / 4);
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

        // ---- log-sum-exp over components, base 2 (lane holds points 4g+r, comp 16b+j)
        float m[4], z[4], e[KB][4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float mx = sc[0][r] + cv[0];
#pragma unroll
            for (int b = 1; b < KB; ++b) mx = fmaxf(mx, sc[b][r] + cv[b]);
            m[r] = row16_max(mx);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float zz = 0.0f;
#pragma unroll
            for (int b = 0; b < KB; ++b) {
                e[b][r] = fast_exp2(sc[b][r] + cv[b] - m[r]);
                zz += e[b][r];
            }
            z[r] = row16_sum(zz);
        }
        const int64_t pbase = t * kTile + w * 16 + 4 * g;
        float lse2[4];
        bool valid[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            lse2[r] = m[r] + fast_log2(z[r]);
            valid[r] = pbase + r < n;
            if (j == 0 && valid[r]) ll2 += (double)lse2[r];
        }

        if constexpr (EM) {
            // ---- responsibilities (registers only), s0, and [s1 | s2] += gamma^T [x | x^2]
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float inv = valid[r] ? 1.0f / z[r] : 0.0f;
#pragma unroll
                for (int b = 0; b < KB; ++b) e[b][r] *= inv;
            }
#pragma unroll
            for (int b = 0; b < KB; ++b) s0acc[b] += (e[b][0] + e[b][1]) + (e[b][2] + e[b][3]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float xv[DP / 16];
                lds_load<DP / 16>(xs + (w * 16 + 4 * g + r) * S::kRow + j * (DP / 16), xv);
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
                        if (sc[b][r] + cv[b] == m[r] && 16 * b + j < k_real) best = 16 * b + j;
                    best = row16_min_i(best);
                    if (j == 0 && valid[r]) out_arg[pbase + r] = best;
                }
            }
        }

        if (t + 1 < t1) ld.store(smem + (cur ^ 1) * kTile * S::kRow);
        __syncthreads();
    }

    // ---- one fp64 partial per workgroup, waves summed in a fixed order
    llred[tid] = ll2;
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
    if constexpr (EM) {
        const int ncol = 1 + 2 * d;
        const float* red = smem;
        for (int e2 = tid; e2 < k_real * ncol; e2 += kThreads) {
            const int k = e2 / ncol, c = e2 % ncol;
            double v = 0.0;
            if (c == 0) {
                for (int w2 = 0; w2 < 4; ++w2)
                    for (int g2 = 0; g2 < 4; ++g2) v += (double)s0red[w2][g2][k];
            } else {   // column 1 + 2 dd + m holds moment m (0: x - c, 1: (x - c)^2) of dim dd
                const int dd = (c - 1) >> 1, mom = (c - 1) & 1;
                const int col = mom * DP + dd;
                for (int w2 = 0; w2 < 4; ++w2) v += (double)red[(w2 * 16 * KB + k) * (2 * DP) + col];
            }
            part[(wg * k_real + k) * ncol + c] = v;
        }
    }
    if (tid == 0) {
        double s = 0.0;
        for (int i = 0; i < kThreads; ++i) s += llred[i];
        part_ll[wg] = s * kLn2;
    }

    // The last workgroup to arrive sums the LL partials in slot order (the
    // order does not depend on which workgroup is last: deterministic).
    __shared__ int is_last;
    __threadfence();
    __syncthreads();
    if (tid == 0) is_last = (atomicAdd(arrivals, 1u) == (unsigned int)(G - 1));
    __syncthreads();
    if (is_last) {
        __threadfence();
        double v = 0.0;
        for (int64_t i = tid; i < G; i += kThreads) v += __builtin_nontemporal_load(part_ll + i);
        v = block_sum_f64(v, llred);
        if (tid == 0) {
            *ll_ws = v;
            if (ll_out) *ll_out = v;
            *nonfinite_ll = isfinite(v) ? 0 : 1;
            *arrivals = 0u;
        }
    }
}

// Per-component preprocessing ([LP-GMM] 3.1, Preprocess): panel columns and
// the log-normaliser of component k from the fp32 parameters in the
// workspace.  Called by all threads of one workgroup.
template <int DP, int KB>
__device__ void prep_component(int k, int d, const float* th_pi, const float* th_mu,
                               const float* th_var, const float* shift, float* panel, float* cvec,
                               int* flags, double* red) {
    double slogv = 0.0, sm2p = 0.0, bad = 0.0;
    for (int dd = threadIdx.x; dd < DP; dd += blockDim.x) {
        float a = 0.0f, b = 0.0f;
        if (dd < d) {
            const double v = th_var[(int64_t)k * d + dd];
            const double mu = (double)th_mu[(int64_t)k * d + dd] - (double)shift[dd];
            if (!(v > 0.0) || !isfinite(v) || !isfinite(mu)) bad += 1.0;
            const double pr = 1.0 / v;
            a = (float)(-0.5 * pr * kLog2e);
            b = (float)(mu * pr * kLog2e);
            slogv += log(v);
            sm2p += mu * mu * pr;
        }
        const int s = dd % (DP / 4), gg = dd / (DP / 4);
        const int ln = gg * 16 + (k & 15), bb = k >> 4;
        panel[((s * 2) * KB + bb) * 64 + ln] = a;
        panel[((s * 2 + 1) * KB + bb) * 64 + ln] = b;
    }
    slogv = block_sum_f64(slogv, red);
    sm2p = block_sum_f64(sm2p, red);
    bad = block_sum_f64(bad, red);
    if (threadIdx.x == 0) {
        const double pk = th_pi[k];
        if (!(pk >= 0.0) || !isfinite(pk)) bad += 1.0;
        const double c = (log(pk) - 0.5 * (d * kLog2Pi + slogv + sm2p)) * kLog2e;
        cvec[k] = (float)c;
        flags[k] = (flags[k] & ~1) | (bad > 0.0 ? 1 : 0);
    }
}

template <int DP, int KB>
__global__ __launch_bounds__(256) void k_diag_prepare(int k_real, int d, const float* pi,
                                                      const float* mu, const float* var,
                                                      float* th_pi, float* th_mu, float* th_var,
                                                      float* shift, float* panel, float* cvec,
                                                      int* flags, unsigned int* arrivals,
                                                      unsigned int* comp_arrivals) {
    __shared__ double red[256];
    __shared__ float csh[DP];
    const int k = blockIdx.x;
    if (k == 0 && threadIdx.x == 0) *arrivals = 0u;
    // centre c = mean of the heaviest component (lowest index on ties): it
    // lies where the data is, unlike a weighted mean that an empty far-away
    // component can drag off.  Every workgroup finds the same one.
    int kstar = 0;
    for (int kk = 1; kk < k_real; ++kk)
        if (pi[kk] > pi[kstar]) kstar = kk;
    for (int dd = threadIdx.x; dd < DP; dd += blockDim.x) {
        const float c = dd < d ? mu[(int64_t)kstar * d + dd] : 0.0f;
        const float cf = isfinite(c) ? c : 0.0f;
        csh[dd] = cf;
        if (k == 0) shift[dd] = cf;
    }
    __syncthreads();
    if (k >= k_real) {  // padding component: zero panel columns, weight 0
        for (int dd = threadIdx.x; dd < DP; dd += blockDim.x) {
            const int s = dd % (DP / 4), gg = dd / (DP / 4);
            const int ln = gg * 16 + (k & 15), bb = k >> 4;
            panel[((s * 2) * KB + bb) * 64 + ln] = 0.0f;
            panel[((s * 2 + 1) * KB + bb) * 64 + ln] = 0.0f;
        }
        if (threadIdx.x == 0) cvec[k] = -INFINITY;
        return;
    }
    for (int dd = threadIdx.x; dd < d; dd += blockDim.x) {
        th_mu[(int64_t)k * d + dd] = mu[(int64_t)k * d + dd];
        th_var[(int64_t)k * d + dd] = var[(int64_t)k * d + dd];
    }
    if (threadIdx.x == 0) {
        th_pi[k] = pi[k];
        flags[k] = 0;               // status bits
        flags[k_real + k] = 0;      // ridge retries (full covariance only)
        comp_arrivals[k] = 0u;
        if (k == 0) flags[2 * k_real] = 0;  // non-finite LL
    }
    __syncthreads();
    prep_component<DP, KB>(k, d, th_pi, th_mu, th_var, csh, panel, cvec, flags, red);
}

// Reduce the per-workgroup partials, M-step, and prepare the next iteration.
// Grid (chunks of 32 dimensions, K).  In workgroup (ch, k), lane l of wave w
// sums column 1 + 64 ch + l over the slots p = w, w + 4, w + 8, ... (fixed
// order), the four waves are combined in order, and threads t < 32 turn the
// moments of dimension 32 ch + t into mu', var', raw moments and panel
// entries.  Per-chunk sums of log var and (mu - c)^2 / var go to a small
// buffer; the last chunk of component k to arrive (atomic counter) combines
// them in chunk order into the log-normaliser c_k and the status flags.
constexpr int kRedChunkDims = 32;

template <int DP, int KB>
__global__ __launch_bounds__(256) void k_diag_reduce_finalize(
    const double* __restrict__ part, int P, int64_t n, int d, int k_real, float var_floor,
    double* __restrict__ stats, float* __restrict__ th_pi, float* __restrict__ th_mu,
    float* __restrict__ th_var, const float* __restrict__ shift, float* __restrict__ out_pi,
    float* __restrict__ out_mu, float* __restrict__ out_var, float* __restrict__ panel,
    float* __restrict__ cvec, int* __restrict__ flags, double* __restrict__ chunk_part,
    unsigned int* __restrict__ comp_arrivals) {
    __shared__ double colw[4][64];
    __shared__ double s0w[256];
    __shared__ double cs[4][kRedChunkDims];
    __shared__ int is_last;
    const int ch = blockIdx.x, k = blockIdx.y, nch = gridDim.x;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int ncol = 1 + 2 * d;
    const int col = 1 + 64 * ch + lane;

    // column sums over the partial slots (4 interleaved accumulators for MLP)
    double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
    if (col < ncol) {
        const double* src = part + (int64_t)k * ncol + col;
        const int64_t stride = (int64_t)k_real * ncol;
        int p = w;
        for (; p + 12 < P; p += 16) {
            a0 += src[(int64_t)p * stride];
            a1 += src[(int64_t)(p + 4) * stride];
            a2 += src[(int64_t)(p + 8) * stride];
            a3 += src[(int64_t)(p + 12) * stride];
        }
        for (; p < P; p += 4) a0 += src[(int64_t)p * stride];
    }
    colw[w][lane] = (a0 + a1) + (a2 + a3);
    // s0: every workgroup of component k sums column 0 the same way
    double z = 0.0;
    for (int p = tid; p < P; p += 256) z += part[((int64_t)p * k_real + k) * ncol];
    const double s0 = block_sum_f64(z, s0w);   // contains __syncthreads
    const bool empty = s0 < kEmptyNk;

    double slogv = 0.0, sm2p = 0.0, bad = 0.0, nonfin = 0.0;
    if (tid < kRedChunkDims) {
        const int dd = kRedChunkDims * ch + tid;
        if (dd < d) {
            const double t1 = (colw[0][2 * tid] + colw[1][2 * tid]) + (colw[2][2 * tid] + colw[3][2 * tid]);
            const double t2 = (colw[0][2 * tid + 1] + colw[1][2 * tid + 1]) +
                              (colw[2][2 * tid + 1] + colw[3][2 * tid + 1]);
            const double c = shift[dd];
            const int64_t i = (int64_t)k * d + dd;
            // raw moments: sum g x = t1 + c s0, sum g x^2 = t2 + 2 c t1 + c^2 s0
            stats[(int64_t)k * ncol + 1 + dd] = t1 + c * s0;
            stats[(int64_t)k * ncol + 1 + d + dd] = t2 + 2.0 * c * t1 + c * c * s0;
            if (!isfinite(t1) || !isfinite(t2)) nonfin += 1.0;
            float mf = th_mu[i], vf = th_var[i];
            if (!empty) {
                const double dm = t1 / s0;
                mf = (float)(c + dm);
                vf = (float)fmax(t2 / s0 - dm * dm, (double)var_floor);
            }
            th_mu[i] = mf;
            th_var[i] = vf;
            if (out_mu) out_mu[i] = mf;
            if (out_var) out_var[i] = vf;
            // next-iteration panel entries from the fp32 parameters
            const double v = vf, mu = (double)mf - c;
            if (!(v > 0.0) || !isfinite(v) || !isfinite(mu)) bad += 1.0;
            const double pr = 1.0 / v;
            const int s = dd % (DP / 4), gg = dd / (DP / 4);
            const int ln = gg * 16 + (k & 15), bb = k >> 4;
            panel[((s * 2) * KB + bb) * 64 + ln] = (float)(-0.5 * pr * kLog2e);
            panel[((s * 2 + 1) * KB + bb) * 64 + ln] = (float)(mu * pr * kLog2e);
            slogv = log(v);
            sm2p = mu * mu * pr;
        }
        cs[0][tid] = slogv;
        cs[1][tid] = sm2p;
        cs[2][tid] = bad;
        cs[3][tid] = nonfin;
    }
    __syncthreads();
    if (tid < 4) {   // fixed-order sum over the chunk's dimensions
        double v = 0.0;
        for (int i = 0; i < kRedChunkDims; ++i) v += cs[tid][i];
        chunk_part[((int64_t)k * nch + ch) * 4 + tid] = v;
    }
    if (tid == 0 && ch == 0) {
        stats[(int64_t)k * ncol] = s0;
        const float pf = (float)(s0 / (double)n);
        th_pi[k] = pf;
        if (out_pi) out_pi[k] = pf;
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) is_last = (atomicAdd(comp_arrivals + k, 1u) == (unsigned int)(nch - 1));
    __syncthreads();
    if (is_last && tid == 0) {
        __threadfence();
        double tot[4] = {0.0, 0.0, 0.0, 0.0};
        for (int c2 = 0; c2 < nch; ++c2)
            for (int q = 0; q < 4; ++q)
                tot[q] += __builtin_nontemporal_load(chunk_part + ((int64_t)k * nch + c2) * 4 + q);
        const double pk = (double)(float)(s0 / (double)n);   // the fp32 pi' just written
        cvec[k] = (float)((log(pk) - 0.5 * (d * kLog2Pi + tot[0] + tot[1])) * kLog2e);
        int f = flags[k] & ~(1 | 4 | 8);
        if (tot[2] > 0.0 || !(pk >= 0.0)) f |= 1;
        if (empty) f |= 4;
        if (tot[3] > 0.0 || !isfinite(s0)) f |= 8;
        flags[k] = f;
        comp_arrivals[k] = 0u;
    }
}

__global__ void k_sum_ll(const double* part_ll, int P, double* ll_ws, double* ll_out,
                         int* nonfinite_ll) {
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        double s = 0.0;
        for (int p = 0; p < P; ++p) s += part_ll[p];
        *ll_ws = s;
        if (ll_out) *ll_out = s;
        *nonfinite_ll = isfinite(s) ? 0 : 1;
    }
}

struct WsPtrs {
    float *pi, *mu, *var, *shift, *panel, *cvec;
    double *part, *part_ll, *stats, *ll;
    int *flags, *retries, *nonfinite_ll;
    unsigned int* arrivals;
    double* chunk_part;
    unsigned int* comp_arrivals;
};

WsPtrs ws_ptrs(const Plan& p, char* ws) {
    WsPtrs w;
    w.pi = (float*)(ws + p.off_pi);
    w.mu = (float*)(ws + p.off_mu);
    w.var = (float*)(ws + p.off_cov);
    w.shift = (float*)(ws + p.off_shift);
    w.panel = (float*)(ws + p.off_panel);
    w.cvec = (float*)(ws + p.off_cvec);
    w.part = (double*)(ws + p.off_part);
    w.part_ll = (double*)(ws + p.off_part_ll);
    w.stats = (double*)(ws + p.off_stats);
    w.ll = (double*)(ws + p.off_ll);
    w.flags = (int*)(ws + p.off_diag);
    w.retries = w.flags + p.k;
    w.nonfinite_ll = w.flags + 2 * p.k;
    w.arrivals = (unsigned int*)(w.flags + 2 * p.k + 1);
    w.chunk_part = (double*)(ws + p.off_chunk);
    w.comp_arrivals = (unsigned int*)(ws + p.off_comp_arrivals);
    return w;
}

template <int DP, int KB, typename XT, bool VEC, bool EM>
hipError_t launch_fused_t(const Plan& p, const WsPtrs& w, const void* x, int grid, int64_t tiles,
                          float* lse, int* arg, double* ll_out, hipStream_t s) {
    hipLaunchKernelGGL((k_diag_fused<DP, KB, XT, VEC, EM>), dim3(grid), dim3(kThreads), 0, s,
                       (const XT*)x, p.n, (int)p.d, p.ldx, (int)p.k, w.panel, w.cvec, w.shift, tiles,
                       w.part, w.part_ll, lse, arg, w.ll, ll_out, w.nonfinite_ll, w.arrivals);
    return hipGetLastError();
}

template <int DP, int KB, bool EM>
hipError_t launch_fused_x(const Plan& p, const WsPtrs& w, const void* x, bool vec, int grid,
                          int64_t tiles, float* lse, int* arg, double* ll_out, hipStream_t s) {
    switch (p.xdt) {
        case GMM_F32:
            return vec ? launch_fused_t<DP, KB, float, true, EM>(p, w, x, grid, tiles, lse, arg, ll_out, s)
                       : launch_fused_t<DP, KB, float, false, EM>(p, w, x, grid, tiles, lse, arg, ll_out, s);
        case GMM_BF16:
            return vec ? launch_fused_t<DP, KB, bf16_t, true, EM>(p, w, x, grid, tiles, lse, arg, ll_out, s)
                       : launch_fused_t<DP, KB, bf16_t, false, EM>(p, w, x, grid, tiles, lse, arg, ll_out, s);
        default:
            return vec ? launch_fused_t<DP, KB, _Float16, true, EM>(p, w, x, grid, tiles, lse, arg, ll_out, s)
                       : launch_fused_t<DP, KB, _Float16, false, EM>(p, w, x, grid, tiles, lse, arg, ll_out, s);
    }
}

#define GMM_DIAG_SHAPES(X) \
    X(16, 1) X(16, 2) X(16, 3) X(16, 4) X(32, 1) X(32, 2) X(32, 3) X(32, 4) X(64, 1) X(64, 2) X(128, 1)

template <bool EM>
hipError_t launch_fused(const Plan& p, const WsPtrs& w, const void* x, bool vec, int grid,
                        int64_t tiles, float* lse, int* arg, double* ll_out, hipStream_t s) {
#define CASE(DP_, KB_) \
    if (p.dp == DP_ && p.kb == KB_) return launch_fused_x<DP_, KB_, EM>(p, w, x, vec, grid, tiles, lse, arg, ll_out, s);
    GMM_DIAG_SHAPES(CASE)
#undef CASE
    return hipErrorInvalidValue;
}

bool x_vec_ok(const Plan& p, const void* x) {
    const int es = p.xdt == GMM_F32 ? 4 : 2;
    const int ev = 16 / es;
    return ((uintptr_t)x % 16 == 0) && ((p.ldx * es) % 16 == 0) && (p.d % ev == 0);
}

}  // namespace

bool diag_shape_supported(int dp, int kb) {
#define CASE(DP_, KB_) if (dp == DP_ && kb == KB_) return true;
    GMM_DIAG_SHAPES(CASE)
#undef CASE
    return false;
}

int diag_grid(const Plan& p) {
    const int64_t tiles = (p.n + kTile - 1) / kTile;
    int64_t g = 2 * (int64_t)device_cu_count();
    if (g > p.p_max) g = p.p_max;
    if (g > tiles) g = tiles;
    return (int)g;
}

gmm_status diag_prepare(const Plan& p, char* ws, const float* pi, const float* mu,
                        const float* var, hipStream_t s) {
    WsPtrs w = ws_ptrs(p, ws);
    hipError_t e = hipErrorInvalidValue;
#define CASE(DP_, KB_)                                                                          \
    if (p.dp == DP_ && p.kb == KB_) {                                                           \
        hipLaunchKernelGGL((k_diag_prepare<DP_, KB_>), dim3(16 * KB_), dim3(256), 0, s, (int)p.k, \
                           (int)p.d, pi, mu, var, w.pi, w.mu, w.var, w.shift, w.panel, w.cvec, w.flags, \
                           w.arrivals, w.comp_arrivals);                                 \
        e = hipGetLastError();                                                                  \
    }
    GMM_DIAG_SHAPES(CASE)
#undef CASE
    return e == hipSuccess ? GMM_OK : GMM_E_HIP;
}

gmm_status diag_em_step(const Plan& p, char* ws, const void* x, double* ll_out, hipStream_t s) {
    WsPtrs w = ws_ptrs(p, ws);
    const int64_t tiles = (p.n + kTile - 1) / kTile;
    const int grid = diag_grid(p);
    hipError_t e = launch_fused<true>(p, w, x, x_vec_ok(p, x), grid, tiles, nullptr, nullptr,
                                      ll_out, s);
    return e == hipSuccess ? GMM_OK : GMM_E_HIP;
}

gmm_status diag_finalize(const Plan& p, char* ws, float* pi, float* mu, float* var,
                         hipStream_t s) {
    WsPtrs w = ws_ptrs(p, ws);
    const int P = diag_grid(p);
    const int nch = (int)((p.d + kRedChunkDims - 1) / kRedChunkDims);
    hipError_t e = hipErrorInvalidValue;
#define CASE(DP_, KB_)                                                                            \
    if (p.dp == DP_ && p.kb == KB_) {                                                             \
        hipLaunchKernelGGL((k_diag_reduce_finalize<DP_, KB_>), dim3(nch, p.k), dim3(256), 0, s,    \
                           w.part, P, p.n, (int)p.d, (int)p.k, p.var_floor, w.stats, w.pi, w.mu,  \
                           w.var, w.shift, pi, mu, var, w.panel, w.cvec, w.flags, w.chunk_part,   \
                           w.comp_arrivals);                                                      \
        e = hipGetLastError();                                                                    \
    }
    GMM_DIAG_SHAPES(CASE)
#undef CASE
    return e == hipSuccess ? GMM_OK : GMM_E_HIP;
}

gmm_status diag_loglik(const Plan& p, char* ws, const void* x, double* ll_out, float* lse,
                       int32_t* argmax, hipStream_t s) {
    WsPtrs w = ws_ptrs(p, ws);
    hipError_t e;
    if (p.n == 0) {
        hipLaunchKernelGGL(k_sum_ll, dim3(1), dim3(64), 0, s, w.part_ll, 0, w.ll, ll_out,
                           w.nonfinite_ll);
        e = hipGetLastError();
    } else {
        const int64_t tiles = (p.n + kTile - 1) / kTile;
        const int grid = diag_grid(p);
        e = launch_fused<false>(p, w, x, x_vec_ok(p, x), grid, tiles, lse, argmax, ll_out, s);
    }
    return e == hipSuccess ? GMM_OK : GMM_E_HIP;
}

}  // namespace gmm
