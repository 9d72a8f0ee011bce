// Diagonal-covariance GMM: parameter preparation, reduction of the fused
// kernel's partials, M-step, and the host entry points of this family.
//
// Preprocess ([LP-GMM] 3.1): per component, the precisions and the score
// panel [a ; b] in the fused kernel's MFMA register layout, plus per-chunk
// (32 dimensions) sums of log sigma^2 and (mu - c)^2 / sigma^2 from which the
// fused kernel forms the log-normaliser c_k itself.  M-step ([Flash-GMM]
// Method, parameter update from s0 / s1 / s2 after one pass): pi' = s0/N,
// mu' = s1/s0, var' = max(s2/s0 - mu'^2, floor), here from moments about the
// fixed centre c so that the subtraction does not cancel.
//
// No kernel here synchronises workgroups with each other: every output has a
// single writer, and consumers run in later kernels on the same stream.

#include "diag_internal.h"

namespace gmm {

namespace {

// Panel entries and per-dimension normaliser terms of component k, dim dd.
struct DimTerms {
    float a, b;
    double logv, m2p, bad;
};

__device__ __forceinline__ DimTerms dim_terms(double var, double mu_c) {
    DimTerms t;
    t.bad = (!(var > 0.0) || !isfinite(var) || !isfinite(mu_c)) ? 1.0 : 0.0;
    const double pr = 1.0 / var;
    t.a = (float)(-0.5 * pr * kLog2e);
    t.b = (float)(mu_c * pr * kLog2e);
    t.logv = log(var);
    t.m2p = mu_c * mu_c * pr;
    return t;
}

template <int DP, int KB>
__device__ __forceinline__ void put_panel(float* panel, int k, int dd, float a, float b) {
    const int s = dd % (DP / 4), gg = dd / (DP / 4);
    const int ln = gg * 16 + (k & 15), bb = k >> 4;
    panel[((s * 2) * KB + bb) * 64 + ln] = a;
    panel[((s * 2 + 1) * KB + bb) * 64 + ln] = b;
}

// gmm_prepare: copy theta into the workspace, choose the centre, build the
// panel and the per-chunk normaliser sums.  Grid: 16*KB workgroups (one per
// padded component), 256 threads.
// Power-of-two scale s of dimension dd for the split-fp16 operands
// y = (x - c) s: the widest reach of the components that hold weight,
// max_k |mu_k - c| + 4 sigma_k over pi_k > 0, maps into [4, 8), so data
// within the model's spread has |y| < 8 and the fp16 range (|y| <
// kSplitLim) leaves a factor of about 28 for points beyond it.  1 when the
// reach is zero or not finite.
template <int KMAX>
__device__ __forceinline__ float dim_scale(int k_real, int d, int dd, float c, const float* pi,
                                           const float* mu, const float* var) {
    // all loads first (clamped, always in bounds) so that they issue together
    float vv[KMAX], mv[KMAX], pv[KMAX];
#pragma unroll
    for (int kk = 0; kk < KMAX; ++kk) {
        const int kc = kk < k_real ? kk : k_real - 1;
        vv[kk] = var[(int64_t)kc * d + dd];
        mv[kk] = mu[(int64_t)kc * d + dd];
        pv[kk] = kk < k_real ? pi[kc] : 0.0f;
    }
    float reach = 0.0f;
#pragma unroll
    for (int kk = 0; kk < KMAX; ++kk) {
        const float r = fabsf(mv[kk] - c) + 4.0f * sqrtf(vv[kk] > 0.0f ? vv[kk] : 0.0f);
        reach = (pv[kk] > 0.0f && isfinite(r)) ? fmaxf(reach, r) : reach;
    }
    if (!(reach > 0.0f) || !isfinite(reach)) return 1.0f;
    int e = ilogbf(reach) - 2;
    e = e < -60 ? -60 : (e > 60 ? 60 : e);
    return ldexpf(1.0f, -e);
}

template <int DP, int KB>
__global__ __launch_bounds__(256) void k_diag_prepare(int k_real, int d, const float* pi,
                                                      const float* mu, const float* var,
                                                      float* th_pi, float* th_mu, float* th_var,
                                                      float* shift, float* panel,
                                                      double* chunk_part, int* flags) {
    __shared__ float csh[DP];
    __shared__ double terms[3][DP];
    const int k = blockIdx.x;
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
    if (k >= k_real) {  // padding component: zero panel columns (its c_k is -inf)
        for (int dd = threadIdx.x; dd < DP; dd += blockDim.x) put_panel<DP, KB>(panel, k, dd, 0.f, 0.f);
        return;
    }
    for (int dd = threadIdx.x; dd < DP; dd += blockDim.x) {
        float a = 0.f, b = 0.f;
        double lv = 0.0, m2 = 0.0, bd = 0.0;
        if (dd < d) {
            const int64_t i = (int64_t)k * d + dd;
            const float vf = var[i], mf = mu[i];
            th_mu[i] = mf;
            th_var[i] = vf;
            const DimTerms t = dim_terms(vf, (double)mf - (double)csh[dd]);
            a = t.a; b = t.b; lv = t.logv; m2 = t.m2p; bd = t.bad;
        }
        put_panel<DP, KB>(panel, k, dd, a, b);
        terms[0][dd] = lv;
        terms[1][dd] = m2;
        terms[2][dd] = bd;
    }
    __syncthreads();
    const int nch = (d + kDiagChunkDims - 1) / kDiagChunkDims;
    if ((int)threadIdx.x < 4 * nch) {   // fixed-order sum over the chunk's dims
        const int ch = threadIdx.x >> 2, q = threadIdx.x & 3;
        double v = 0.0;
        if (q < 3)
            for (int t = 0; t < kDiagChunkDims; ++t) {
                const int dd = ch * kDiagChunkDims + t;
                if (dd < d) v += terms[q][dd];
            }
        chunk_part[((int64_t)k * nch + ch) * 4 + q] = v;
    }
    if (threadIdx.x == 0) {
        const float pk = pi[k];
        th_pi[k] = pk;
        flags[k] = (!(pk >= 0.0f) || !isfinite(pk)) ? 1 : 0;   // bit 0: bad weight
        flags[k_real + k] = 0;                                 // ridge retries (full only)
        if (k == 0) flags[2 * k_real] = 0;                     // non-finite LL
    }
}

// Split fp16 panel of the split kernel from the prepared fp32 parameters
// (after gmm_prepare and after every finalize): the per-dimension scale s
// (every workgroup derives the same one; workgroup 0 stores it for the
// reduction of the coming step), and the entries
// a_kd = -1/2 log2(e) / (var s^2) and b_kd = log2(e) (mu - c) / (var s)
// (y units), divided by the component's power of two F_k that puts its
// largest entry in [2^14, 2^15), each stored as hi = fp16(v), lo = fp16(v - hi)
// in the B-operand layout of v_mfma_f32_16x16x32_f16: contraction index kk
// (a at kk = dd, b at kk = DP + dd) of component k sits in k-step kk / 32,
// block k / 16, lane 16 ((kk % 32) / 8) + k % 16, half kk % 8.  Padding
// components and dimensions get zeros (F = 1).  Grid: 16 KB workgroups (one
// per padded component), DP threads.
template <int DP, int KB>
__global__ __launch_bounds__(DP) void k_diag_split_panel(int k_real, int d, const float* th_pi,
                                                         const float* th_mu, const float* th_var,
                                                         const float* shift, float* scale,
                                                         const double* chunk_part, int nch,
                                                         uint16_t* panel16, float* fk, float* ck) {
    __shared__ float red[DP];
    const int k = blockIdx.x, dd = threadIdx.x;
    const float sd = dd < d ? dim_scale<16 * KB>(k_real, d, dd, shift[dd], th_pi, th_mu, th_var) : 1.0f;
    if (k == 0) scale[dd] = sd;
    double a = 0.0, b = 0.0;
    if (k < k_real && dd < d) {
        const int64_t i = (int64_t)k * d + dd;
        const double s = sd;
        const double pr = 1.0 / (double)th_var[i];
        a = -0.5 * pr * kLog2e / (s * s);
        b = ((double)th_mu[i] - (double)shift[dd]) * pr * kLog2e / s;
    }
    const float m = (float)fmax(fabs(a), fabs(b));
    red[dd] = isfinite(m) ? m : 0.0f;
    __syncthreads();
    for (int st = DP / 2; st > 0; st >>= 1) {
        if (dd < st) red[dd] = fmaxf(red[dd], red[dd + st]);
        __syncthreads();
    }
    const float mx = red[0];
    const int fe = mx > 0.0f ? ilogbf(mx) - 14 : 0;
    const double inv = ldexp(1.0, -fe);
    constexpr size_t kLo = (size_t)(DP / 16) * KB * 64 * 8;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int kk = h * DP + dd;
        const float v = (float)((h == 0 ? a : b) * inv);
        const _Float16 hi = (_Float16)v;
        const _Float16 lo = (_Float16)(v - (float)hi);
        const size_t o = ((size_t)((kk / 32) * KB + k / 16) * 64 + 16 * ((kk % 32) / 8) + k % 16) * 8 + kk % 8;
        panel16[o] = __builtin_bit_cast(uint16_t, hi);
        panel16[kLo + o] = __builtin_bit_cast(uint16_t, lo);
    }
    if (dd == 0) {
        fk[k] = ldexpf(1.0f, fe);
        // c_k = log2(e) (log pi_k - 1/2 (D log 2pi + sum log var + sum (mu-c)^2/var)),
        // from the per-chunk sums of the prepare / finalize kernel
        float c = -INFINITY;   // padding component: weight 0
        if (k < k_real) {
            double sl = 0.0, sm = 0.0;
            for (int ch = 0; ch < nch; ++ch) {
                sl += chunk_part[((int64_t)k * nch + ch) * 4 + 0];
                sm += chunk_part[((int64_t)k * nch + ch) * 4 + 1];
            }
            c = (float)((log((double)th_pi[k]) - 0.5 * (d * kLog2Pi + sl + sm)) * kLog2e);
        }
        ck[k] = c;
    }
}

// Reduce the per-workgroup partials, M-step, and prepare the next iteration.
// Grid (chunks of 32 dimensions, K).  In workgroup (ch, k), lane l of wave w
// sums column 1 + 64 ch + l over the slots p = w, w + 4, w + 8, ... (fixed
// order), the four waves are combined in order, and threads t < 32 turn the
// moments of dimension 32 ch + t into mu', var', raw moments and panel
// entries.  The chunk's sums of log var and (mu - c)^2 / var (and counts of
// bad / non-finite values) go to chunk_part[k][ch]; the next fused kernel
// forms c_k from them.
template <int DP, int KB>
__global__ __launch_bounds__(256) void k_diag_reduce_finalize(
    const double* __restrict__ part, int P, int64_t n, int d, int k_real, float var_floor,
    double* __restrict__ stats, float* __restrict__ th_pi, float* __restrict__ th_mu,
    float* __restrict__ th_var, const float* __restrict__ shift, const float* __restrict__ scale,
    float* __restrict__ out_pi,
    float* __restrict__ out_mu, float* __restrict__ out_var, float* __restrict__ panel,
    int* __restrict__ flags, double* __restrict__ chunk_part) {
    __shared__ double colw[4][64];
    __shared__ double s0w[256];
    __shared__ double cs[4][kDiagChunkDims];
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
    if (tid < kDiagChunkDims) {
        const int dd = kDiagChunkDims * ch + tid;
        if (dd < d) {
            // moments of y = (x - c) s back to x - c (s is a power of two: exact)
            const double is = 1.0 / (double)scale[dd];
            const double t1 = ((colw[0][2 * tid] + colw[1][2 * tid]) + (colw[2][2 * tid] + colw[3][2 * tid])) * is;
            const double t2 = ((colw[0][2 * tid + 1] + colw[1][2 * tid + 1]) +
                               (colw[2][2 * tid + 1] + colw[3][2 * tid + 1])) * is * is;
            const double c = shift[dd];
            const int64_t i = (int64_t)k * d + dd;
            // raw moments: sum g x = t1 + c s0, sum g x^2 = t2 + 2 c t1 + c^2 s0
            stats[(int64_t)k * ncol + 1 + dd] = t1 + c * s0;
            stats[(int64_t)k * ncol + 1 + d + dd] = t2 + 2.0 * c * t1 + c * c * s0;
            if (!isfinite(t1) || !isfinite(t2)) nonfin = 1.0;
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
            const DimTerms t = dim_terms(vf, (double)mf - c);
            put_panel<DP, KB>(panel, k, dd, t.a, t.b);
            slogv = t.logv;
            sm2p = t.m2p;
            bad = t.bad;
        }
        cs[0][tid] = slogv;
        cs[1][tid] = sm2p;
        cs[2][tid] = bad;
        cs[3][tid] = nonfin;
    }
    __syncthreads();
    if (tid < 4) {   // fixed-order sum over the chunk's dimensions
        double v = 0.0;
        for (int i = 0; i < kDiagChunkDims; ++i) v += cs[tid][i];
        chunk_part[((int64_t)k * nch + ch) * 4 + tid] = v;
    }
    if (tid == 0 && ch == 0) {
        stats[(int64_t)k * ncol] = s0;
        const float pf = (float)(s0 / (double)n);
        th_pi[k] = pf;
        if (out_pi) out_pi[k] = pf;
        int f = 0;
        if (!(pf >= 0.0f) || !isfinite(pf)) f |= 1 | 8;
        if (empty) f |= 4;
        flags[k] = f;
    }
}

// LL of the fused kernel: fixed-order sum of the per-workgroup partials.
__global__ __launch_bounds__(256) void k_sum_ll(const double* part_ll, int P, double* ll_ws,
                                                double* ll_out, int* nonfinite_ll) {
    __shared__ double red[256];
    double v = 0.0;
    for (int p = threadIdx.x; p < P; p += 256) v += part_ll[p];
    v = block_sum_f64(v, red);
    if (threadIdx.x == 0) {
        *ll_ws = v;
        if (ll_out) *ll_out = v;
        *nonfinite_ll = isfinite(v) ? 0 : 1;
    }
}

}  // namespace

bool diag_shape_supported(int dp, int kb) {
#define CASE(DP_, KB_) if (dp == DP_ && kb == KB_) return true;
    GMM_DIAG_SHAPES(CASE)
#undef CASE
    return false;
}

int diag_grid(const Plan& p) {
    const int64_t groups = (p.n + 31) / 32;                     // 32-point tiles
    const int64_t per_wg = diag_split_waves(p.dp, p.kb);        // at least one per wave
    int64_t g = (int64_t)kDiagWgPerCu * device_cu_count();
    if (g > p.p_max) g = p.p_max;
    const int64_t need = (groups + per_wg - 1) / per_wg;
    if (g > need) g = need;
    return (int)(g < 1 ? 1 : g);
}

gmm_status diag_prepare(const Plan& p, char* ws, const float* pi, const float* mu,
                        const float* var, hipStream_t s) {
    DiagWs w = diag_ws(p, ws);
    hipError_t e = hipErrorInvalidValue;
#define CASE(DP_, KB_)                                                                          \
    if (p.dp == DP_ && p.kb == KB_) {                                                           \
        hipLaunchKernelGGL((k_diag_prepare<DP_, KB_>), dim3(16 * KB_), dim3(256), 0, s, (int)p.k, \
                           (int)p.d, pi, mu, var, w.pi, w.mu, w.var, w.shift, w.panel,           \
                           w.chunk_part, w.flags);                                               \
        hipLaunchKernelGGL((k_diag_split_panel<DP_, KB_>), dim3(16 * KB_), dim3(DP_), 0, s,      \
                           (int)p.k, (int)p.d, w.pi, w.mu, w.var, w.shift, w.scale,             \
                           w.chunk_part, diag_chunks(p), (uint16_t*)w.panel16, w.fk, w.ck);     \
        e = hipGetLastError();                                                                  \
    }
    GMM_DIAG_SHAPES(CASE)
#undef CASE
    return e == hipSuccess ? GMM_OK : GMM_E_HIP;
}

static gmm_status sum_ll(const Plan& p, const DiagWs& w, int P, double* ll_out, hipStream_t s) {
    hipLaunchKernelGGL(k_sum_ll, dim3(1), dim3(256), 0, s, w.part_ll, P, w.ll, ll_out,
                       w.nonfinite_ll);
    return hipGetLastError() == hipSuccess ? GMM_OK : GMM_E_HIP;
}

gmm_status diag_em_step(const Plan& p, char* ws, const void* x, double* ll_out, hipStream_t s) {
    DiagWs w = diag_ws(p, ws);
    const int P = diag_grid(p);
    hipError_t e = diag_launch_split(p, w, x, true, P, nullptr, nullptr, s);
    if (e != hipSuccess) return GMM_E_HIP;
    return sum_ll(p, w, P, ll_out, s);
}

gmm_status diag_finalize(const Plan& p, char* ws, float* pi, float* mu, float* var,
                         hipStream_t s) {
    DiagWs w = diag_ws(p, ws);
    const int P = diag_grid(p);
    const int nch = diag_chunks(p);
    hipError_t e = hipErrorInvalidValue;
#define CASE(DP_, KB_)                                                                            \
    if (p.dp == DP_ && p.kb == KB_) {                                                             \
        hipLaunchKernelGGL((k_diag_reduce_finalize<DP_, KB_>), dim3(nch, p.k), dim3(256), 0, s,    \
                           w.part, P, p.n, (int)p.d, (int)p.k, p.var_floor, w.stats, w.pi, w.mu,  \
                           w.var, w.shift, w.scale, pi, mu, var, w.panel, w.flags, w.chunk_part); \
        hipLaunchKernelGGL((k_diag_split_panel<DP_, KB_>), dim3(16 * KB_), dim3(DP_), 0, s,        \
                           (int)p.k, (int)p.d, w.pi, w.mu, w.var, w.shift, w.scale,               \
                           w.chunk_part, diag_chunks(p), (uint16_t*)w.panel16, w.fk, w.ck);       \
        e = hipGetLastError();                                                                    \
    }
    GMM_DIAG_SHAPES(CASE)
#undef CASE
    return e == hipSuccess ? GMM_OK : GMM_E_HIP;
}

gmm_status diag_loglik(const Plan& p, char* ws, const void* x, double* ll_out, float* lse,
                       int32_t* argmax, hipStream_t s) {
    DiagWs w = diag_ws(p, ws);
    if (p.n == 0) return sum_ll(p, w, 0, ll_out, s);
    const int P = diag_grid(p);
    hipError_t e = diag_launch_split(p, w, x, false, P, lse, argmax, s);
    if (e != hipSuccess) return GMM_E_HIP;
    return sum_ll(p, w, P, ll_out, s);
}

}  // namespace gmm
