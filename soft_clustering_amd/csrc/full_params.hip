// Full-covariance family: batched ridged Cholesky (parameter preparation),
// reduction of the fused kernel's partials, M-step, and the host entry points.
//
// Preparation ([LP-GMM] 3.1 Preprocess; 1.2 route 2; 4.1 ridge; 2.1 storage):
// per component C~ = C + eps I with eps = ridge_rel |tr C| / D, L = chol(C~)
// in fp64; on a pivot that is not positive (or not finite) eps becomes
// max(10 eps, 1e-3 |tr C| / D) and the factorisation is repeated, at most 3
// times, after which the component is flagged not positive definite and its
// weight is treated as 0.  The forward solve L z = x - mu is carried out by
// the fused kernel as a product with W = (L 2^-e_k)^{-1} (2^e_k near
// sqrt(|tr C|/D)), which this kernel forms in fp64 (a triangular inverse,
// one row per step) and stores as a split fp16 panel (hi + lo, 22
// bits) with the bias W mu; log|C~| = 2 sum log L_ii from the fp64 factor.
// The mean is also stored in fp16 as the centre of the second moments.
// M-step ([Flash-GMM] Method): pi' = s0/N, mu' = s1/s0,
// C' = sum gamma (x - mu')(x - mu')^T / s0, here from the second moment
// about the stored centre: C' = M2/s0 - delta delta^T, delta = mu' - centre.
// A component with s0 < 1e-6 keeps its mean and covariance.

#include <math.h>
#include <string.h>

#include "full_internal.h"

namespace gmm {

namespace {

// 1 / x from the hardware estimate and two Newton steps (each doubles the
// number of correct bits: about 2^-26 -> 2^-52 -> the last bit).  Used on the
// factorisation's pivots; what it yields for a pivot that is not positive or
// not finite is discarded, as the factorisation stops on such a pivot.
__device__ __forceinline__ double recip_f64(double x) {
    double r = __builtin_amdgcn_rcp(x);
    r = fma(r, fma(-x, r, 1.0), r);
    r = fma(r, fma(-x, r, 1.0), r);
    return r;
}

constexpr int kRidgeRetries = 3;
constexpr double kRidgeEscalate = 1e-3;   // escalation floor, relative to |tr C| / D

__global__ __launch_bounds__(256) void k_full_load(int k_real, int d, const float* pi,
                                                   const float* mu, const float* cov, float* th_pi,
                                                   float* th_mu, float* th_cov, int* flags) {
    const int k = blockIdx.x;
    for (int i = threadIdx.x; i < d * d; i += blockDim.x)
        th_cov[(int64_t)k * d * d + i] = cov[(int64_t)k * d * d + i];
    for (int i = threadIdx.x; i < d; i += blockDim.x) th_mu[(int64_t)k * d + i] = mu[(int64_t)k * d + i];
    if (threadIdx.x == 0) {
        const float pk = pi[k];
        th_pi[k] = pk;
        flags[k] = (!(pk >= 0.0f) || !isfinite(pk)) ? 1 : 0;
        flags[k_real + k] = 0;
        if (k == 0) flags[2 * k_real] = flags[2 * k_real + 1] = 0;
    }
}

// One workgroup per padded component (TG x TG threads: 16 x 16, or 32 x 32 at
// D = 128).  The factorisation is right-looking on the lower triangle of C~
// (fp64), one column per step: each thread holds its elements
// (ti + TG a, tc + TG b) in registers and the column of each step is
// broadcast through LDS.
template <int DP, int TG>
__global__ __launch_bounds__(TG * TG) void k_full_chol(int k_real, int d, float ridge_rel,
                                                   const float* pi, const float* mu,
                                                   const float* cov, uint4* wpk, float* wbias,
                                                   float* muh, float* cvec, float* rscale,
                                                   int* flags) {
    constexpr int NOB = full_nob(DP), NKS = full_nks(DP), DPO = full_dpo(DP);
    constexpr int NV = 2 * NOB * NKS * 64;   // panel vectors per component
    constexpr int NT = TG * TG;
    constexpr int RT = DP / TG;   // rows (and columns) of the matrix per thread
    __shared__ double A[DP][DP + 1];   // C~, then its factor; at the end W = (L s)^{-1}
    double(*W)[DP + 1] = A;           // (one matrix of LDS: 132 KB at D = 128)
    __shared__ double pinv[DP], mus[DP];
    __shared__ double pan[2][4][DP];   // four broadcast columns (factorisation), double-buffered
    __shared__ double rpan[2][4][DP];  // four broadcast rows (inverse), double-buffered
    __shared__ double red[NT];
    const int k = blockIdx.x, tid = threadIdx.x;
    const int ti = tid / TG, tc = tid % TG;   // this thread's elements: (ti + TG a, tc + TG b)
    uint4* Wk = wpk + (int64_t)k * NV;
    auto put_identity = [&]() {   // a zero panel: the component is never scored (c_k = -inf)
        for (int i = tid; i < NV; i += NT) Wk[i] = make_uint4(0, 0, 0, 0);
        for (int i = tid; i < DPO; i += NT) wbias[k * DPO + i] = 0.0f;
        for (int i = tid; i < DP; i += NT) muh[k * DP + i] = 0.0f;
        if (tid == 0) {
            cvec[k] = -INFINITY;
            rscale[k] = 1.0f;
        }
    };
    if (k >= k_real) {   // padding component
        put_identity();
        return;
    }
    const float* C = cov + (int64_t)k * d * d;
    // this thread's elements of the lower triangle, |trace| / D and the
    // bad-parameter check (non-finite entries of the lower triangle)
    float Cr[RT][RT];
    double tr = 0.0, bad = 0.0;
#pragma unroll
    for (int a = 0; a < RT; ++a)
#pragma unroll
        for (int b2 = 0; b2 < RT; ++b2) {
            const int r = ti + TG * a, c = tc + TG * b2;
            const bool in = c <= r && r < d;
            Cr[a][b2] = in ? C[(int64_t)r * d + c] : 0.0f;
            if (in && !isfinite(Cr[a][b2])) bad = 1.0;
            if (in && r == c) tr += (double)Cr[a][b2];
        }
    tr = block_sum_f64(tr, red);
    bad = block_sum_f64(bad, red);
    const double scale = fabs(tr) / (double)d;
    double eps = (double)ridge_rel * scale;
    int attempt = 0;
    bool ok = false;
    double Ar[RT][RT];
    for (; attempt <= kRidgeRetries; ++attempt) {
#pragma unroll
        for (int a = 0; a < RT; ++a)
#pragma unroll
            for (int b2 = 0; b2 < RT; ++b2) {
                const int r = ti + TG * a, c = tc + TG * b2;
                double v = 0.0;
                if (c <= r) {
                    if (r < d) v = (double)Cr[a][b2] + (r == c ? eps : 0.0);
                    else v = (r == c) ? 1.0 : 0.0;   // padded dimensions: identity
                }
                Ar[a][b2] = v;
            }
        // Blocked by 4 columns: step st takes columns J = 4 st .. 4 st + 3.  Every
        // thread factors the 4 x 4 diagonal block itself (pivots p_t, multipliers
        // l_tu = x'_u(j0 + t) / p_u), maps the panel values x_u(r) = A_r,j0+u of
        // its rows and columns to x'(r) (x'_t = x_t - sum_{u<t} l_tu x'_u: what the
        // four single-column steps would leave), and updates
        // A_ic -= sum_t x'_t(i) x'_t(c) / p_t for c > j0 + 3, c <= i.  The owners
        // of J keep x' (the unscaled factor: L_ij = x'_j(i) / sqrt(p_j)); the owners
        // of the next four columns publish them (final at the start of the next
        // step) into the other half of the double-buffered panel.
        if (tc < 4) {
#pragma unroll
            for (int a = 0; a < RT; ++a) pan[0][tc][ti + TG * a] = Ar[a][0];
        }
        bool failed = false;
        for (int st = 0; st < DP / 4; ++st) {
            const int j0 = 4 * st;
            __syncthreads();
            const double(*pv)[DP] = pan[st & 1];
            double p[4], rp[4], l[4][4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                double xs[4];
#pragma unroll
                for (int u = 0; u <= t; ++u) {
                    double v = pv[u][j0 + t];
#pragma unroll
                    for (int w2 = 0; w2 < u; ++w2) v -= l[u][w2] * xs[w2];
                    xs[u] = v;
                    if (u < t) l[t][u] = v * rp[u];
                }
                p[t] = xs[t];
                rp[t] = recip_f64(p[t]);
            }
            bool bad_piv = false;   // the same in every thread: the test is uniform
#pragma unroll
            for (int t = 0; t < 4; ++t) bad_piv = bad_piv || !(p[t] > 0.0) || !isfinite(p[t]);
            if (bad_piv) {
                failed = true;
                break;
            }
            auto transform = [&](int r, double (&xo)[4]) __attribute__((always_inline)) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    double v = pv[u][r];
#pragma unroll
                    for (int w2 = 0; w2 < u; ++w2) v -= l[u][w2] * xo[w2];
                    xo[u] = v;
                }
            };
            double xc[RT][4];
#pragma unroll
            for (int b2 = 0; b2 < RT; ++b2) transform(tc + TG * b2, xc[b2]);
            const int own_t = tc - (j0 % TG);   // column j0 + own_t is this thread's (0..3)
#pragma unroll
            for (int a = 0; a < RT; ++a) {
                const int i = ti + TG * a;
                double xr[4];
                transform(i, xr);
                if (i > j0 + 3) {
                    double g[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) g[t] = xr[t] * rp[t];
#pragma unroll
                    for (int b2 = 0; b2 < RT; ++b2) {
                        const int c = tc + TG * b2;
                        if (c > j0 + 3 && c <= i)
                            Ar[a][b2] -= g[0] * xc[b2][0] + g[1] * xc[b2][1] + g[2] * xc[b2][2] +
                                         g[3] * xc[b2][3];
                    }
                }
                if (own_t >= 0 && own_t < 4 && i >= j0 + own_t) {
                    double v = xr[0];
#pragma unroll
                    for (int t = 1; t < 4; ++t)
                        if (own_t == t) v = xr[t];
#pragma unroll
                    for (int b2 = 0; b2 < RT; ++b2)
                        if (b2 == j0 / TG) Ar[a][b2] = v;
                }
            }
            const int jn = j0 + 4, nt = tc - (jn % TG);
            if (jn < DP && nt >= 0 && nt < 4) {
#pragma unroll
                for (int b2 = 0; b2 < RT; ++b2)
                    if (b2 == jn / TG) {
#pragma unroll
                        for (int a = 0; a < RT; ++a) pan[(st + 1) & 1][nt][ti + TG * a] = Ar[a][b2];
                    }
            }
        }
        __syncthreads();
        if (!failed) {
            ok = true;
            break;
        }
        eps = fmax(10.0 * eps, kRidgeEscalate * scale);
    }
    if (!ok || bad > 0.0) {
        put_identity();
        if (tid == 0) {
            flags[k] |= (bad > 0.0 ? 1 : 0) | (ok ? 0 : 2);
            flags[k_real + k] = attempt > kRidgeRetries ? kRidgeRetries : attempt;
        }
        return;
    }
#pragma unroll
    for (int a = 0; a < RT; ++a)
#pragma unroll
        for (int b2 = 0; b2 < RT; ++b2) A[ti + TG * a][tc + TG * b2] = Ar[a][b2];
    // scale s = 2^-e with 2^e near sqrt(|tr| / D)
    int e = 0;
    if (scale > 0.0 && isfinite(scale)) {
        e = ilogb(sqrt(scale));
        e = e < -60 ? -60 : (e > 60 ? 60 : e);
    }
    const double sc = ldexp(1.0, -e);
    // W = (L s)^{-1}, L = U D^{1/2} with U unit lower triangular (U_ij = A_ij / A_jj):
    // W = s^-1 D^{-1/2} U^{-1}.  U^{-1} right-looking from R = I: once row i of R is
    // final, the rows below take R_r -= U_ri R_i.
    __syncthreads();
    for (int i = tid; i < DP; i += NT) {
        pinv[i] = 1.0 / A[i][i];
        mus[i] = i < d ? (double)mu[(int64_t)k * d + i] : 0.0;
    }
    double Rr[RT][RT];
#pragma unroll
    for (int a = 0; a < RT; ++a)
#pragma unroll
        for (int b2 = 0; b2 < RT; ++b2) Rr[a][b2] = (ti + TG * a == tc + TG * b2) ? 1.0 : 0.0;
    // blocked by 4 rows: step st takes rows I = 4 st .. 4 st + 3 (their values y at
    // the start of the step broadcast through rpan).  Every thread finishes the
    // block rows for its columns (y'_t = y_t - sum_{w<t} U_{i0+t, i0+w} y'_w), the
    // owners of I keep y', and the rows below take R_r -= sum_t U_{r, i0+t} y'_t.
    if (ti < 4) {
#pragma unroll
        for (int b2 = 0; b2 < RT; ++b2) rpan[0][ti][tc + TG * b2] = Rr[0][b2];
    }
    for (int st = 0; st < DP / 4; ++st) {
        const int i0 = 4 * st;
        __syncthreads();
        const double(*rv)[DP] = rpan[st & 1];
        double ub[4][4];   // U within the block
#pragma unroll
        for (int t = 1; t < 4; ++t)
#pragma unroll
            for (int w2 = 0; w2 < t; ++w2) ub[t][w2] = A[i0 + t][i0 + w2] * pinv[i0 + w2];
        double yc[RT][4];
#pragma unroll
        for (int b2 = 0; b2 < RT; ++b2) {
            const int c = tc + TG * b2;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                double v = rv[t][c];
#pragma unroll
                for (int w2 = 0; w2 < t; ++w2) v -= ub[t][w2] * yc[b2][w2];
                yc[b2][t] = v;
            }
        }
        const int own_t = ti - (i0 % TG);   // row i0 + own_t is this thread's (0..3)
#pragma unroll
        for (int a = 0; a < RT; ++a) {
            const int r = ti + TG * a;
            if (r > i0 + 3) {
                double ur[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) ur[t] = A[r][i0 + t] * pinv[i0 + t];
#pragma unroll
                for (int b2 = 0; b2 < RT; ++b2)
                    Rr[a][b2] -= ur[0] * yc[b2][0] + ur[1] * yc[b2][1] + ur[2] * yc[b2][2] +
                                 ur[3] * yc[b2][3];
            } else if (own_t >= 0 && own_t < 4 && a == i0 / TG) {
#pragma unroll
                for (int b2 = 0; b2 < RT; ++b2) {
                    double v = yc[b2][0];
#pragma unroll
                    for (int t = 1; t < 4; ++t)
                        if (own_t == t) v = yc[b2][t];
                    Rr[a][b2] = v;
                }
            }
        }
        const int in = i0 + 4, nt = ti - (in % TG);
        if (in < DP && nt >= 0 && nt < 4) {
#pragma unroll
            for (int a = 0; a < RT; ++a)
                if (a == in / TG) {
#pragma unroll
                    for (int b2 = 0; b2 < RT; ++b2) rpan[(st + 1) & 1][nt][tc + TG * b2] = Rr[a][b2];
                }
        }
    }
    __syncthreads();
    // log|C~| = 2 sum log L_ii from the fp64 factor, before W takes its place
    double ld = 0.0;
    for (int i = tid; i < d; i += NT) ld += 0.5 * log(A[i][i]);   // log L_ii
    ld = block_sum_f64(ld, red);
    // W = (L s)^{-1}; where its largest entry would leave the range the fp16
    // panel holds comfortably (above 2^14: a covariance far wider in one
    // direction than its mean variance suggests), s grows by the power of two
    // that brings the largest entry into [2^13, 2^14)
    double wmax = 0.0;
#pragma unroll
    for (int a = 0; a < RT; ++a) {
        const int r = ti + TG * a;
        const double f = sqrt(pinv[r]) / sc;   // 1 / (sqrt(A_rr) s)
#pragma unroll
        for (int b2 = 0; b2 < RT; ++b2) {
            Rr[a][b2] *= f;
            wmax = fmax(wmax, fabs(Rr[a][b2]));
        }
    }
    red[tid] = wmax;
    __syncthreads();
    for (int s2 = NT / 2; s2 > 0; s2 >>= 1) {
        if (tid < s2) red[tid] = fmax(red[tid], red[tid + s2]);
        __syncthreads();
    }
    wmax = red[0];
    const int e2 = (wmax > 16384.0 && isfinite(wmax)) ? ilogb(wmax) - 13 : 0;
    const double sc2 = ldexp(sc, e2), wf = ldexp(1.0, -e2);
#pragma unroll
    for (int a = 0; a < RT; ++a)
#pragma unroll
        for (int b2 = 0; b2 < RT; ++b2) W[ti + TG * a][tc + TG * b2] = Rr[a][b2] * wf;
    __syncthreads();
    // panel: out dimension o = 32 ob + l % 32 (rows), input i = 16 ks + 8 (l / 32) + q;
    // zero outside the D x D lower triangle; hi = fp16(w), lo = fp16(w - hi)
    for (int v = tid; v < NV / 2; v += NT) {
        const int l = v % 64, ks = (v / 64) % NKS, ob = v / (64 * NKS);
        const int o = 32 * ob + (l & 31);
        uint32_t hw[4], lw[4];
        for (int q2 = 0; q2 < 4; ++q2) {
            _Float16 h[2], lo[2];
            for (int t = 0; t < 2; ++t) {
                const int ic = 16 * ks + 8 * (l >> 5) + 2 * q2 + t;
                const double wv = (o < d && ic < d && ic <= o) ? W[o][ic] : 0.0;
                const float fv = (float)wv;
                h[t] = (_Float16)fv;
                lo[t] = (_Float16)(fv - (float)h[t]);
            }
            hw[q2] = (uint32_t)__builtin_bit_cast(uint16_t, h[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, h[1]) << 16);
            lw[q2] = (uint32_t)__builtin_bit_cast(uint16_t, lo[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, lo[1]) << 16);
        }
        Wk[v] = make_uint4(hw[0], hw[1], hw[2], hw[3]);              // hi half of the panel
        Wk[NV / 2 + v] = make_uint4(lw[0], lw[1], lw[2], lw[3]);     // lo half
    }
    // bias W mu (fp64), the fp16 centre of the moments
    for (int o = tid; o < DPO; o += NT) {
        double bsum = 0.0;
        if (o < d)
            for (int ic = 0; ic <= o; ++ic) bsum += W[o][ic] * mus[ic];
        wbias[k * DPO + o] = (float)bsum;
    }
    for (int i = tid; i < DP; i += NT) muh[k * DP + i] = (float)(_Float16)(float)mus[i];
    if (tid == 0) {
        const double logdet = 2.0 * ld;
        const double lp = log((double)pi[k]);
        cvec[k] = (float)(kLog2e * (lp - 0.5 * ((double)d * kLog2Pi + logdet)));
        rscale[k] = (float)sc2;
        if (bad > 0.0) flags[k] |= 1;
        flags[k_real + k] = attempt;
    }
}

// Column sums (fp64) of the fp32 partials over the workgroups, fixed order.
// Grid (ceil(ncolp / 64), K); thread (c, q) of a workgroup sums the quarter q of
// the workgroups for column c in four interleaved chains, and the quarters are
// added in a fixed order.
__global__ __launch_bounds__(256) void k_full_reduce(const float* __restrict__ part, int P,
                                                     int ncolp, double* __restrict__ colsum,
                                                     int add) {
    __shared__ double qs[4][64];
    const int k = blockIdx.y, c = threadIdx.x % 64, q = threadIdx.x / 64;
    const int col = blockIdx.x * 64 + c;
    const int64_t stride = (int64_t)kFullKP * ncolp;
    const int pq = (P + 3) / 4, p0 = q * pq, p1 = p0 + pq < P ? p0 + pq : P;
    double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
    if (col < ncolp) {
        const float* src = part + (int64_t)k * ncolp + col;
        int i = p0;
        for (; i + 3 < p1; i += 4) {
            a0 += (double)src[(int64_t)i * stride];
            a1 += (double)src[(int64_t)(i + 1) * stride];
            a2 += (double)src[(int64_t)(i + 2) * stride];
            a3 += (double)src[(int64_t)(i + 3) * stride];
        }
        for (; i < p1; ++i) a0 += (double)src[(int64_t)i * stride];
    }
    qs[q][c] = (a0 + a1) + (a2 + a3);
    __syncthreads();
    if (q == 0 && col < ncolp) {
        const double v = (qs[0][c] + qs[1][c]) + (qs[2][c] + qs[3][c]);
        double* o = colsum + (int64_t)k * ncolp + col;
        *o = add ? *o + v : v;   // add: a later segment of the same pass
    }
}

// M-step per component (grid K, 256 threads) and the raw statistics
// [s0, s1 (D), sum gamma x x^T (D x D)].
__global__ __launch_bounds__(256) void k_full_mstep(const double* __restrict__ colsum, int64_t n,
                                                    int d, int dp, const float* __restrict__ muh,
                                                    double* __restrict__ stats,
                                                    float* __restrict__ th_pi,
                                                    float* __restrict__ th_mu,
                                                    float* __restrict__ th_cov, float* out_pi,
                                                    float* out_mu, float* out_cov, int* flags) {
    __shared__ double red[256];
    __shared__ double cen[128], s1v[128], dlt[128];   // centre, s1, mu' - centre (d <= 128)
    const int k = blockIdx.x, tid = threadIdx.x;
    const int ncolp = 1 + d + d * (d + 1) / 2;
    const double* cs = colsum + (int64_t)k * ncolp;
    const double s0 = cs[0];
    const bool empty = !(s0 >= kEmptyNk);
    const double is0 = 1.0 / s0;
    double* st = stats + (int64_t)k * (1 + d + (int64_t)d * d);
    double nonfin = isfinite(s0) ? 0.0 : 1.0;
    for (int i = tid; i < d; i += 256) {
        const double s1 = cs[1 + i];
        const double ci = muh[k * dp + i];
        cen[i] = ci;
        s1v[i] = s1;
        dlt[i] = s1 * is0 - ci;
        st[1 + i] = s1;
        if (!isfinite(s1)) nonfin = 1.0;
        float mf = th_mu[(int64_t)k * d + i];
        if (!empty) mf = (float)(s1 * is0);
        th_mu[(int64_t)k * d + i] = mf;
        if (out_mu) out_mu[(int64_t)k * d + i] = mf;
    }
    __syncthreads();
    // row i = q / d from a float estimate (exact here: q < 128^2 and the quotient's
    // distance to the next integer is at least 1 / (2 d))
    const float inv_d = 1.0f / (float)d;
#pragma unroll 4
    for (int q = tid; q < d * d; q += 256) {
        const int i = (int)(((float)q + 0.5f) * inv_d), c = q - i * d;
        const int r0 = i > c ? i : c, c0 = i > c ? c : i;
        const double m2 = cs[1 + d + tri_idx(r0, c0)];     // about the stored centre
        const double ci = cen[i], cc = cen[c];
        // raw moment: sum g x x^T = M2 + c s1^T + s1 c^T - s0 c c^T
        st[1 + d + q] = m2 + ci * s1v[c] + s1v[i] * cc - s0 * ci * cc;
        if (!isfinite(m2)) nonfin = 1.0;
        float v = th_cov[(int64_t)k * d * d + q];
        if (!empty) v = (float)(m2 * is0 - dlt[i] * dlt[c]);
        th_cov[(int64_t)k * d * d + q] = v;
        if (out_cov) out_cov[(int64_t)k * d * d + q] = v;
    }
    nonfin = block_sum_f64(nonfin, red);
    if (tid == 0) {
        st[0] = s0;
        const float pf = (float)(s0 / (double)n);
        th_pi[k] = pf;
        if (out_pi) out_pi[k] = pf;
        int f = flags[k] & 2;   // not-PD status of the parameters this pass used
        if (!(pf >= 0.0f) || !isfinite(pf)) f |= 1 | 8;
        if (nonfin > 0.0) f |= 8;
        if (empty) f |= 4;
        flags[k] = f;
    }
}

__global__ __launch_bounds__(256) void k_full_sum_ll(const double* part_ll, int P, double* ll_ws,
                                                     double* ll_out, int* misc) {
    __shared__ double red[256];
    double v = 0.0;
    for (int q = threadIdx.x; q < P; q += 256) v += part_ll[q];
    v = block_sum_f64(v, red);
    if (threadIdx.x == 0) {
        *ll_ws = v;
        if (ll_out) *ll_out = v;
        misc[0] = isfinite(v) ? 0 : 1;
    }
}

// Several groups: per point the natural-log LSE over the groups' LSEs
// (written over row 0), the LL partial of each workgroup (fixed order), and
// for the E-step the caller's LSE and argmax (lowest component on ties: the
// first group whose largest score is the overall largest).
__global__ __launch_bounds__(256) void k_full_merge(int64_t n, int G, float* glse, const int* garg,
                                                    const float* gmax, double* part_ll,
                                                    float* out_lse, int* out_arg) {
    __shared__ double red[256];
    constexpr float kL2e = 1.44269504088896340736f, kLn2f = 0.69314718055994530942f;
    double ll = 0.0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < n; p += stride) {
        float M = -INFINITY;
        for (int g = 0; g < G; ++g) M = fmaxf(M, glse[(int64_t)g * n + p]);
        const float Ms = M == -INFINITY ? 0.0f : M;
        float Z = 0.0f;
        for (int g = 0; g < G; ++g) Z += fast_exp2((glse[(int64_t)g * n + p] - Ms) * kL2e);
        const float lse = Ms + fast_log2(Z) * kLn2f;
        glse[p] = lse;
        ll += (double)lse;
        if (out_lse) out_lse[p] = lse;
        if (out_arg) {
            float bm = -INFINITY;
            int a = 0;
            for (int g = 0; g < G; ++g) {
                const float v = gmax[(int64_t)g * n + p];
                if (v > bm) {
                    bm = v;
                    a = garg[(int64_t)g * n + p];
                }
            }
            out_arg[p] = a;
        }
    }
    ll = block_sum_f64(ll, red);
    if (threadIdx.x == 0) part_ll[blockIdx.x] = ll;
}

int merge_grid(const Plan& p) {
    int64_t g = (p.n + 255) / 256;
    if (g > kFullLLSlots) g = kFullLLSlots;
    return (int)(g < 1 ? 1 : g);
}

FullPass pass_of(int g) {
    FullPass ps;
    memset(&ps, 0, sizeof(ps));
    ps.group = g;
    return ps;
}

// Several groups, first loop: every group's LSE per point (and, on request,
// its argmax and largest score), then the merge.
hipError_t group_lse(const Plan& p, const FullWs& w, const void* x, float* out_lse, int* out_arg,
                     hipStream_t s) {
    const int G = full_grid(p);
    const int64_t tiles = (p.n + kFullT - 1) / kFullT;
    for (int g = 0; g < w.groups; ++g) {
        FullPass ps = pass_of(g);
        ps.out_lse = w.glse + (size_t)g * p.n;
        if (out_arg) {
            ps.out_arg = w.garg + (size_t)g * p.n;
            ps.out_max = w.gmax + (size_t)g * p.n;
        }
        const hipError_t e = full_launch_fused(p, w, x, false, G, ps, 0, tiles, 1, s);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_full_merge, dim3(merge_grid(p)), dim3(256), 0, s, p.n, w.groups, w.glse,
                       (const int*)w.garg, (const float*)w.gmax, w.part_ll, out_lse, out_arg);
    return hipGetLastError();
}

hipError_t chol(const Plan& p, const FullWs& w, hipStream_t s) {
#define FULL_CHOL(DP_, TG_)                                                                       \
    hipLaunchKernelGGL((k_full_chol<DP_, TG_>), dim3(kFullKP * w.groups), dim3(TG_ * TG_), 0, s,     \
                       (int)p.k, (int)p.d, p.ridge_rel, w.pi, w.mu, w.cov, w.wpk, w.wbias, w.muh,    \
                       w.cvec, w.rscale, w.flags)
    switch (p.dp) {
        case 16: FULL_CHOL(16, 16); break;
        case 32: FULL_CHOL(32, 16); break;
        case 64: FULL_CHOL(64, 16); break;
        case 128: FULL_CHOL(128, 32); break;
        default: return hipErrorInvalidValue;
    }
#undef FULL_CHOL
    return hipGetLastError();
}

gmm_status sum_ll(const Plan& p, const FullWs& w, int P, double* ll_out, hipStream_t s) {
    hipLaunchKernelGGL(k_full_sum_ll, dim3(1), dim3(256), 0, s, w.part_ll, P, w.ll, ll_out,
                       w.flags + 2 * p.k);
    return hipGetLastError() == hipSuccess ? GMM_OK : GMM_E_HIP;
}

}  // namespace

gmm_status full_prepare(const Plan& p, char* ws, const float* pi, const float* mu,
                        const float* cov, hipStream_t s) {
    FullWs w = full_ws(p, ws);
    hipLaunchKernelGGL(k_full_load, dim3(p.k), dim3(256), 0, s, (int)p.k, (int)p.d, pi, mu, cov,
                       w.pi, w.mu, w.cov, w.flags);
    if (hipGetLastError() != hipSuccess) return GMM_E_HIP;
    return chol(p, w, s) == hipSuccess ? GMM_OK : GMM_E_HIP;
}

// Reduce group g's partial slots into its components' column sums (add:
// onto the sums of the earlier segments of the same pass).
hipError_t reduce_group(const Plan& p, const FullWs& w, int g, int P, int add, hipStream_t s) {
    const int ncolp = (int)full_ncolp(p.d);
    const int64_t k0 = (int64_t)kFullKP * g;
    const int kc = (int)(p.k - k0 < kFullKP ? p.k - k0 : kFullKP);
    hipLaunchKernelGGL(k_full_reduce, dim3((ncolp + 63) / 64, kc), dim3(256), 0, s,
                       w.part + (size_t)g * w.slots * kFullKP * ncolp, P, ncolp,
                       w.colsum + k0 * ncolp, add);
    return hipGetLastError();
}

gmm_status full_em_step(const Plan& p, char* ws, const void* x, double* ll_out, hipStream_t s) {
    FullWs w = full_ws(p, ws);
    const int G = full_grid(p);
    const FullSegs sg = full_segs(p, G);
    const bool many = w.lse_pass;
    if (many && group_lse(p, w, x, nullptr, nullptr, s) != hipSuccess) return GMM_E_HIP;
    for (int g = 0; g < w.groups; ++g) {
        FullPass ps = pass_of(g);
        ps.lse_in = many ? w.glse : nullptr;   // second loop: normalise with the merged LSE
        // D > 64: one statistics launch per quad of live components
        const int64_t kc = p.k - (int64_t)kFullKP * g < kFullKP ? p.k - (int64_t)kFullKP * g : kFullKP;
        const int nq = p.dp > 64 ? (int)((kc + 3) / 4) : 1;
        for (int i = 0; i < sg.n; ++i) {
            const int64_t lo = (int64_t)i * sg.len, hi = lo + sg.len < sg.tiles ? lo + sg.len : sg.tiles;
            for (int q = 0; q < nq; ++q) {
                ps.quad = q;
                if (full_launch_fused(p, w, x, true, G, ps, lo, hi, i == 0, s) != hipSuccess) return GMM_E_HIP;
            }
            // every segment but the last is closed here; finalize adds the last one
            if (i + 1 < sg.n && reduce_group(p, w, g, G, i > 0 ? 1 : 0, s) != hipSuccess) return GMM_E_HIP;
        }
    }
    return sum_ll(p, w, many ? merge_grid(p) : G, ll_out, s);
}

gmm_status full_finalize(const Plan& p, char* ws, float* pi, float* mu, float* cov,
                         hipStream_t s) {
    FullWs w = full_ws(p, ws);
    const int G = full_grid(p);
    const int add = full_segs(p, G).n > 1 ? 1 : 0;
    for (int g = 0; g < w.groups; ++g)
        if (reduce_group(p, w, g, G, add, s) != hipSuccess) return GMM_E_HIP;
    hipLaunchKernelGGL(k_full_mstep, dim3(p.k), dim3(256), 0, s, w.colsum, p.n, (int)p.d, p.dp,
                       w.muh, w.stats, w.pi, w.mu, w.cov, pi, mu, cov, w.flags);
    if (hipGetLastError() != hipSuccess) return GMM_E_HIP;
    return chol(p, w, s) == hipSuccess ? GMM_OK : GMM_E_HIP;
}

gmm_status full_loglik(const Plan& p, char* ws, const void* x, double* ll_out, float* lse,
                       int32_t* argmax, hipStream_t s) {
    FullWs w = full_ws(p, ws);
    if (p.n == 0) return sum_ll(p, w, 0, ll_out, s);
    if (w.lse_pass) {
        if (group_lse(p, w, x, lse, argmax, s) != hipSuccess) return GMM_E_HIP;
        return sum_ll(p, w, merge_grid(p), ll_out, s);
    }
    const int G = full_grid(p);
    FullPass ps = pass_of(0);
    ps.out_lse = lse;
    ps.out_arg = argmax;
    if (full_launch_fused(p, w, x, false, G, ps, 0, (p.n + kFullT - 1) / kFullT, 1, s) != hipSuccess)
        return GMM_E_HIP;
    return sum_ll(p, w, G, ll_out, s);
}

gmm_status full_assign(const Plan& p, char* ws, const void* x, int m, int32_t* idx, float* gamma,
                       double* ll_out, hipStream_t s) {
    FullWs w = full_ws(p, ws);
    if (p.n == 0) return sum_ll(p, w, 0, ll_out, s);
    const int G = full_grid(p);
    const bool many = w.lse_pass;
    if (many && group_lse(p, w, x, nullptr, nullptr, s) != hipSuccess) return GMM_E_HIP;
    for (int g = 0; g < w.groups; ++g) {   // the groups in order, merging into the lists
        FullPass ps = pass_of(g);
        ps.lse_in = many ? w.glse : nullptr;
        ps.topm = m;
        ps.out_idx = idx;
        ps.out_gamma = gamma;
        ps.tm_first = g == 0;
        ps.tm_last = g == w.groups - 1;
        if (full_launch_fused(p, w, x, false, G, ps, 0, (p.n + kFullT - 1) / kFullT, 1, s) != hipSuccess)
            return GMM_E_HIP;
    }
    return sum_ll(p, w, many ? merge_grid(p) : G, ll_out, s);
}

}  // namespace gmm
