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
        if (k == 0) {
            flags[2 * k_real] = 0;       // non-finite LL
            flags[2 * k_real + 1] = 0;   // finished-workgroup count of the fused kernel
        }
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
__global__ __launch_bounds__(kDiagReduceThreads) void k_diag_reduce_finalize(
    const double* __restrict__ part, int P, int64_t n, int d, int k_real, float var_floor,
    double* __restrict__ stats, float* __restrict__ th_pi, float* __restrict__ th_mu,
    float* __restrict__ th_var, const float* __restrict__ shift, const float* __restrict__ scale,
    float* __restrict__ out_pi,
    float* __restrict__ out_mu, float* __restrict__ out_var, float* __restrict__ panel,
    int* __restrict__ flags, double* __restrict__ chunk_part) {
    constexpr int RW = kDiagReduceThreads / 64;   // waves
    __shared__ double colw[RW][64];
    __shared__ double s0w[kDiagReduceThreads];
    __shared__ double cs[4][kDiagChunkDims];
    const int ch = blockIdx.x, k = blockIdx.y, nch = gridDim.x;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int ncol = 1 + 2 * d;
    const int col = 1 + 64 * ch + lane;

    // column sums over the partial slots: wave w takes slots w, w + RW, ...
    // (4 interleaved accumulators, so that several loads are in flight)
    double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
    if (col < ncol) {
        const double* src = part + (int64_t)k * ncol + col;
        const int64_t stride = (int64_t)k_real * ncol;
        int p = w;
        for (; p + 3 * RW < P; p += 4 * RW) {
            a0 += src[(int64_t)p * stride];
            a1 += src[(int64_t)(p + RW) * stride];
            a2 += src[(int64_t)(p + 2 * RW) * stride];
            a3 += src[(int64_t)(p + 3 * RW) * stride];
        }
        for (; p < P; p += RW) a0 += src[(int64_t)p * stride];
    }
    colw[w][lane] = (a0 + a1) + (a2 + a3);
    // s0: every workgroup of component k sums column 0 the same way
    double z = 0.0;
    for (int p = tid; p < P; p += kDiagReduceThreads) z += part[((int64_t)p * k_real + k) * ncol];
    const double s0 = block_sum_f64(z, s0w);   // contains __syncthreads
    // the waves' column sums, in a fixed order
    auto colsum = [&](int c2) {
        double v = 0.0;
#pragma unroll
        for (int ww = 0; ww < RW; ++ww) v += colw[ww][c2];
        return v;
    };
    const bool empty = s0 < kEmptyNk;

    double slogv = 0.0, sm2p = 0.0, bad = 0.0, nonfin = 0.0;
    if (tid < kDiagChunkDims) {
        const int dd = kDiagChunkDims * ch + tid;
        if (dd < d) {
            // moments of y = (x - c) s back to x - c (s is a power of two: exact)
            const double is = 1.0 / (double)scale[dd];
            const double t1 = colsum(2 * tid) * is;
            const double t2 = colsum(2 * tid + 1) * is * is;
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
    hipError_t e = diag_launch_split(p, w, x, true, P, ll_out, nullptr, nullptr, DiagTopm{0, nullptr, nullptr}, s);
    return e == hipSuccess ? GMM_OK : GMM_E_HIP;
}

gmm_status diag_finalize(const Plan& p, char* ws, float* pi, float* mu, float* var,
                         hipStream_t s) {
    DiagWs w = diag_ws(p, ws);
    const int P = diag_grid(p);
    const int nch = diag_chunks(p);
    hipError_t e = hipErrorInvalidValue;
#define CASE(DP_, KB_)                                                                            \
    if (p.dp == DP_ && p.kb == KB_) {                                                             \
        hipLaunchKernelGGL((k_diag_reduce_finalize<DP_, KB_>), dim3(nch, p.k), dim3(kDiagReduceThreads), 0, s, \
                           w.part, P, p.n, (int)p.d, (int)p.k, p.var_floor, w.stats, w.pi, w.mu,  \
                           w.var, w.shift, w.scale, pi, mu, var, w.panel, w.flags, w.chunk_part); \
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
    hipError_t e = diag_launch_split(p, w, x, false, P, ll_out, lse, argmax, DiagTopm{0, nullptr, nullptr}, s);
    return e == hipSuccess ? GMM_OK : GMM_E_HIP;
}

gmm_status diag_assign(const Plan& p, char* ws, const void* x, int m, int32_t* idx, float* gamma,
                       double* ll_out, hipStream_t s) {
    DiagWs w = diag_ws(p, ws);
    if (p.n == 0) return sum_ll(p, w, 0, ll_out, s);
    const int P = diag_grid(p);
    hipError_t e = diag_launch_split(p, w, x, false, P, ll_out, nullptr, nullptr, DiagTopm{m, idx, gamma}, s);
    return e == hipSuccess ? GMM_OK : GMM_E_HIP;
}

}  // namespace gmm
