// Large-K family: parameter preparation, the slice merge of the two-sweep
// log-sum-exp, reduction of the fused kernel's partials, M-step, and the host
// entry points.
//
// Preprocess ([LP-GMM] 3.1): per component the precisions, the fp16 score
// panel and the log-normaliser, here in base 2 and with power-of-two scales
// (per dimension on X, per component on the panel) chosen so that every fp16
// operand is in range.  The centre and the per-dimension scale come from a
// sample of X, so they are set at the start of every pass over X (em_step,
// loglik), and the panel is rebuilt then from the current theta.  M-step ([Flash-GMM] Method, parameter update):
// pi' = s0/N, mu' = s1/s0, var' = max(s2/s0 - mu'^2, floor) per dimension
// (diagonal) or max((s2/s0 - |mu'|^2) / D, floor) (isotropic), evaluated from
// moments about the centre c used by the fused kernel.  A component with
// s0 < 1e-6 keeps its mean and variance.
//
// Every output has a single writer; kernels never wait on each other except
// through stream order.

#include <math.h>
#include <string.h>

#include "largek_internal.h"

namespace gmm {

namespace {

constexpr int kKpw = 4;   // components per workgroup in the panel kernel (one per wave)

__device__ __forceinline__ double wave_sum_f64(double v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ double wave_max_f64(double v) {
    for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
    return v;
}

// gmm_prepare, step 1: copy theta into the workspace and reset the flags.
// Grid K, 128 threads.
__global__ __launch_bounds__(128) void k_lk_load(int k_real, int d, bool iso, const float* pi,
                                                 const float* mu, const float* var, float* th_pi,
                                                 float* th_mu, float* th_var, int* flags, int* xc_pos,
                                                 int* xc_n) {
    const int k = blockIdx.x;
    for (int dd = threadIdx.x; dd < d; dd += blockDim.x) {
        th_mu[(int64_t)k * d + dd] = mu[(int64_t)k * d + dd];
        if (!iso) th_var[(int64_t)k * d + dd] = var[(int64_t)k * d + dd];
    }
    if (threadIdx.x == 0) {
        const float pk = pi[k];
        th_pi[k] = pk;
        if (iso) th_var[k] = var[k];
        flags[k] = (!(pk >= 0.0f) || !isfinite(pk)) ? 1 : 0;
        flags[k_real + k] = 0;
        xc_pos[k] = -1;   // no exactly scored component until a pass lists them
        if (k == 0) {
            flags[2 * k_real] = 0;
            flags[2 * k_real + 1] = 0;
            *xc_n = 0;
        }
    }
}

// Sample of X for the centre and scale: up to kLkScanRows rows spread evenly
// over N; workgroup b scans sample rows [b * R, (b + 1) * R), R = rows per
// workgroup.  Thread t handles dimension t % DP for rows t / DP, t / DP +
// 256 / DP, ...  Output per (workgroup, dim): (sum, min, max), fixed order.
template <bool BF16>
__global__ __launch_bounds__(256) void k_lk_scan(const uint16_t* __restrict__ x, int64_t n,
                                                 int64_t ldx, int d, int dp, float* scan) {
    __shared__ float red[3][256];
    const int tid = threadIdx.x, dd = tid % dp, ph = tid / dp, nph = 256 / dp;
    const int64_t ns = n < kLkScanRows ? n : kLkScanRows;
    const int per = kLkScanRows / kLkScanWgs;
    float sum = 0.0f, lo = INFINITY, hi = -INFINITY;
    if (dd < d) {
#pragma unroll 8
        for (int i = blockIdx.x * per + ph; i < (blockIdx.x + 1) * per && i < ns; i += nph) {
            const int64_t row = (int64_t)i * n / ns;
            const uint32_t b = x[row * ldx + dd];
            float v;
            if constexpr (BF16) v = __uint_as_float(b << 16);
            else v = (float)__builtin_bit_cast(_Float16, (uint16_t)b);
            if (isfinite(v)) {
                sum += v;
                lo = fminf(lo, v);
                hi = fmaxf(hi, v);
            }
        }
    }
    red[0][tid] = sum;
    red[1][tid] = lo;
    red[2][tid] = hi;
    __syncthreads();
    if (tid < dp) {
        float s = 0.0f, l = INFINITY, h = -INFINITY;
        for (int q = 0; q < nph; ++q) {
            s += red[0][q * dp + tid];
            l = fminf(l, red[1][q * dp + tid]);
            h = fmaxf(h, red[2][q * dp + tid]);
        }
        float* o = scan + ((int64_t)blockIdx.x * dp + tid) * 3;
        o[0] = s;
        o[1] = l;
        o[2] = h;
    }
}

// Centre and per-dimension scale of X for the fused kernel, from the scan:
// c_d = sample mean of the finite values rounded to the storage type, s_d =
// 2^-e_d with 2^e_d the power of two at or below 1/8 of the sample's largest
// |x_d - c_d|, so the sampled y' lie in [-16, 16] and y'^2 stays below the
// fp16 maximum for |y'| < 255.  Isotropic: 2^-g with the sampled bound of
// |x - c|^2 times 2^-g below 2^14, so |y|^2 2^-g stays in fp16 range for
// points within twice the sampled spread.  One workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void k_lk_centre(int64_t n, int d, int dp, bool bf16, bool iso,
                                                    const float* scan, float2* dsc, float* prm) {
    // thread (part, dd): dimension dd = tid % 128 over the scan workgroups
    // b = part (mod 8); the eight parts combined in a fixed tree through LDS
    constexpr int kParts = 8;
    static_assert(kLkScanWgs % kParts == 0, "scan workgroups in groups of eight");
    __shared__ double red[1024];
    __shared__ double ps[kParts][128];
    __shared__ float plo[kParts][128], phi[kParts][128];
    const int dd = threadIdx.x % 128, part = threadIdx.x / 128;
    if (dd < d) {
        double s = 0.0;
        float lo = INFINITY, hi = -INFINITY;
#pragma unroll 8
        for (int b = part; b < kLkScanWgs; b += kParts) {
            const float* o = scan + ((int64_t)b * dp + dd) * 3;
            s += (double)o[0];
            lo = fminf(lo, o[1]);
            hi = fmaxf(hi, o[2]);
        }
        ps[part][dd] = s;
        plo[part][dd] = lo;
        phi[part][dd] = hi;
    }
    __syncthreads();
    double r2 = 0.0;
    if (part == 0 && dd < d) {
        const int64_t ns = n < kLkScanRows ? n : kLkScanRows;
        const double s = ((ps[0][dd] + ps[1][dd]) + (ps[2][dd] + ps[3][dd])) +
                         ((ps[4][dd] + ps[5][dd]) + (ps[6][dd] + ps[7][dd]));
        float lo = plo[0][dd], hi = phi[0][dd];
#pragma unroll
        for (int q = 1; q < kParts; ++q) {
            lo = fminf(lo, plo[q][dd]);
            hi = fmaxf(hi, phi[q][dd]);
        }
        // c is rounded to X's storage type, so x - c is exact in fp32 and, for
        // data within ~2^11 storage ulps of c, exact in fp16 too: no rounding
        // bias shared by every point of a coarse storage lattice
        double c = (ns > 0 && isfinite(s)) ? s / (double)ns : 0.0;
        if (bf16) c = (double)(float)(__bf16)(float)c;
        else if (fabs(c) < 65504.0) c = (double)(float)(_Float16)(float)c;
        const double r = fmax((double)hi - c, c - (double)lo);
        int e = 0;
        if (r > 0.0 && isfinite(r)) {
            e = ilogb(r) - 3;
            e = e < -60 ? -60 : (e > 60 ? 60 : e);
            r2 = r * r;
        }
        dsc[dd] = make_float2((float)c, (float)ldexp(1.0, -e));
    } else if (part == 0 && dd < dp) {
        dsc[dd] = make_float2(0.0f, 0.0f);
    }
    r2 = block_sum_f64(r2, red);
    if (threadIdx.x == 0) {
        int g = 0;
        if (iso && r2 > 0.0 && isfinite(r2)) {
            g = ilogb(r2) - 13;
            g = g < -100 ? -100 : (g > 100 ? 100 : g);
        }
        prm[1] = (float)ldexp(1.0, -g);
        prm[2] = (float)ldexp(1.0, g);
    }
}

// Score panel of one component per wave (grid Kpad / 4, 256 threads), lane
// l handling dimensions l and l + 64.  Contraction index i (inner):
//   diag: [0, DP) A_k (multiplies y'^2), [DP, 2 DP) B_k (multiplies y'),
//         2 DP + {0, 1}: C_k high / low parts (against ones);
//   iso:  [0, DP) W_k (multiplies y'), DP + {0, 1, 2}: P_k 2^g high, high, low
//         (against |y|^2 2^-g high, low, high), DP + {3, 4}: C_k high / low;
// all multiplied by 2^-f, one power of two for every component, chosen so the
// largest magnitude of any component lies in [2^13, 2^14).  Entry (i, k)
// lives at half index ((i / 16 * nblk + k / 32) * 64 + k % 32 + 32 * (i % 16 / 8)) * 8 + i % 8,
// the A-operand register layout of v_mfma_f32_32x32x16_f16 (lane l holds row
// l % 32, K values 8 (l / 32) .. + 7).  Padding components: zero entries and
// C_k = -inf.  Pass 0 writes each component's largest magnitude, the flags
// and nothing else; pass 1 derives 2^-f from all of them and writes the panel.
template <bool WRITE>
__global__ __launch_bounds__(256) void k_lk_panel(int k_real, int kpad, int d, int dp, bool iso,
                                                  int nblk, const float* pi, const float* mu,
                                                  const float* var, const float2* dsc, float* kmax,
                                                  float* prm, uint16_t* panel, int* flags, float* c0,
                                                  const int* xc_pos) {
    __shared__ float red[256];
    const int lane = threadIdx.x & 63;
    const int k = blockIdx.x * kKpw + (threadIdx.x >> 6);
    const int inner = (iso ? dp : 2 * dp) + 16;
    double sc = 1.0;
    if constexpr (WRITE) {
        float mx = 0.0f;   // over the components the panel scores (not the exact ones)
        for (int i = threadIdx.x; i < kpad; i += 256)
            if (i >= k_real || xc_pos[i] < 0) mx = fmaxf(mx, kmax[i]);
        red[threadIdx.x] = mx;
        __syncthreads();
        for (int o = 128; o > 0; o >>= 1) {
            if ((int)threadIdx.x < o) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + o]);
            __syncthreads();
        }
        const float M = red[0];
        int f = 0;
        if (M > 0.0f && isfinite(M)) f = ilogb(M) - 13;
        sc = ldexp(1.0, -f);
        if (blockIdx.x == 0 && threadIdx.x == 0) prm[0] = (float)ldexp(1.0, f);
    }
    auto put = [&](int i, double v) {
        const _Float16 h = (_Float16)(float)v;
        const int64_t idx = (((int64_t)(i / 16) * nblk + k / 32) * 64 + k % 32 + 32 * ((i % 16) / 8)) * 8 + i % 8;
        panel[idx] = __builtin_bit_cast(uint16_t, h);
    };
    auto put_bias = [&](double c, double pg) {   // the 16 bias slots (lanes 0..15)
        if (lane >= 16) return;
        const int b = iso ? dp : 2 * dp;
        double v = 0.0;
        // high part, and the remainder when the high part is finite
        const double ch = (double)(float)(_Float16)(float)c, ph = (double)(float)(_Float16)(float)pg;
        const double cl = isfinite(ch) ? c - ch : 0.0, pl = isfinite(ph) ? pg - ph : 0.0;
        if (iso) {
            if (lane == 0 || lane == 1) v = ph;
            else if (lane == 2) v = pl;
            else if (lane == 3) v = ch;
            else if (lane == 4) v = cl;
        } else {
            if (lane == 0) v = ch;
            else if (lane == 1) v = cl;
        }
        put(b + lane, v);
    };
    // padding component, or one scored in the exact centred form instead:
    // zero panel entries, score -inf
    if (k >= k_real || (WRITE && xc_pos[k] >= 0)) {
        if constexpr (WRITE) {
            for (int i = lane; i < inner - 16; i += 64) put(i, 0.0);
            put_bias(-INFINITY, 0.0);
        } else if (lane == 0) {
            kmax[k] = 0.0f;
            c0[k] = -INFINITY;
        }
        return;
    }
    const double g2 = (double)prm[2];   // 2^g (isotropic |y|^2 scale)
    // unscaled panel entries (fp64) for dims lane, lane + 64
    double ea[2] = {0.0, 0.0}, eb[2] = {0.0, 0.0};
    double logv = 0.0, m2p = 0.0, mx = 0.0, bad = 0.0, err2 = 0.0, yt2 = 0.0;
    const double vi = iso ? (double)var[k] : 0.0;
    for (int h = 0; h < 2; ++h) {
        const int dd = lane + 64 * h;
        if (dd >= d) continue;
        const double v = iso ? vi : (double)var[(int64_t)k * d + dd];
        const double c = dsc[dd].x, esc = 1.0 / (double)dsc[dd].y;   // 2^e_d
        const double mc = (double)mu[(int64_t)k * d + dd] - c;
        if (!(v > 0.0) || !isfinite(v) || !isfinite(mc)) bad = 1.0;
        const double pr = 1.0 / v;
        // |y| of a point near this component: |mu - c| + 3 sigma
        const double yt = fabs(mc) + 3.0 * sqrt(fabs(v));
        yt2 += yt * yt;
        if (iso) {
            ea[h] = kLog2e * mc * pr * esc;                 // W
            mx = fmax(mx, fabs(ea[h]));
            err2 += (kLog2e * mc * pr * yt) * (kLog2e * mc * pr * yt);
        } else {
            ea[h] = -0.5 * kLog2e * pr * esc * esc;         // A (multiplies y'^2)
            eb[h] = kLog2e * mc * pr * esc;                 // B (multiplies y')
            mx = fmax(mx, fmax(fabs(ea[h]), fabs(eb[h])));
            logv += log(v);
            const double ta = 0.5 * kLog2e * pr * yt * yt, tb = kLog2e * mc * pr * yt;
            err2 += ta * ta + tb * tb;
        }
        m2p += mc * mc * pr;
    }
    logv = wave_sum_f64(logv);
    m2p = wave_sum_f64(m2p);
    mx = wave_max_f64(mx);
    bad = wave_max_f64(bad);
    err2 = wave_sum_f64(err2);
    yt2 = wave_sum_f64(yt2);
    if (iso) logv = (double)d * log(vi);
    const double lp = log((double)pi[k]);
    const double cst = kLog2e * (lp - 0.5 * ((double)d * kLog2Pi + logv + m2p));   // C_k (base 2)
    const double cct = kLog2e * (lp - 0.5 * ((double)d * kLog2Pi + logv));          // centred form
    const double pg = iso ? -0.5 * kLog2e / vi * g2 : 0.0;                         // P_k 2^g
    if constexpr (!WRITE) {
        if (lane == 0) {
            double m = mx;
            if (isfinite(cst)) m = fmax(m, fabs(cst));
            m = fmax(m, fabs(pg));
            kmax[k] = isfinite(m) ? (float)m : 0.0f;
            c0[k] = (float)cct;
            int f = flags[k] & ~16;   // the conditioning flag describes this theta only
            if (bad > 0.0) f |= 1;
            // rounding-error estimate of the fp16 expanded score near the mean,
            // nats: two roundings of relative size <= 2^-11 per panel term
            // (random signs), the 2^-22 split of C_k and of P_k |y|^2
            const double e2 = sqrt(err2) * ldexp(1.0, -11) * (1.41421356 / 1.7320508) +
                              fabs(cst) * ldexp(1.0, -22) + fabs(pg / g2) * yt2 * ldexp(1.0, -21);
            if (e2 * kLn2 > kLkIllCondNats && bad == 0.0 && isfinite(cst)) f |= 16;
            flags[k] = f;
        }
    } else {
        for (int h = 0; h < 2; ++h) {
            const int dd = lane + 64 * h;
            if (dd >= dp) continue;
            put(dd, ea[h] * sc);
            if (!iso) put(dp + dd, eb[h] * sc);
        }
        put_bias(cst * sc, pg * sc);
    }
}

// Two-sweep merge: per point, the base-2 LSE over the slices (written over
// slice 0's entry), LL partial per workgroup (fixed order), and for the
// E-step alone the natural-log LSE and the argmax (lowest component on ties:
// the first slice whose maximum is the overall maximum).
__global__ __launch_bounds__(256) void k_lk_merge(int64_t n, int S, float* part_lse,
                                                  const int* part_arg, const float* part_max,
                                                  double* part_ll, float* out_lse, int* out_arg,
                                                  const int* xc_n) {
    __shared__ double red[256];
    double ll = 0.0;
    // rows: the S slices, and row S when components are scored exactly
    const int R = S + (*xc_n > 0 ? 1 : 0);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < n; p += stride) {
        // every row's value first (all loads in flight), then the combine
        constexpr int kMaxRows = 4096 / kLkSlice + 1;
        float v[kMaxRows];
        float M = -INFINITY;
#pragma unroll
        for (int s = 0; s < kMaxRows; ++s)
            if (s < R) v[s] = part_lse[(int64_t)s * n + p];
#pragma unroll
        for (int s = 0; s < kMaxRows; ++s)
            if (s < R) M = fmaxf(M, v[s]);
        const float Ms = M == -INFINITY ? 0.0f : M;
        float Z = 0.0f;
#pragma unroll
        for (int s = 0; s < kMaxRows; ++s)
            if (s < R) Z += fast_exp2(v[s] - Ms);
        const float lse = Ms + fast_log2(Z);
        part_lse[p] = lse;
        ll += (double)lse;
        if (out_lse) out_lse[p] = lse * (float)kLn2;
        if (out_arg) {
            float bm = -INFINITY;
            int arg = 0x7FFFFFFF;
            for (int s = 0; s < R; ++s) {
                const float v = part_max[(int64_t)s * n + p];
                const int a = part_arg[(int64_t)s * n + p];
                if (v > bm || (v == bm && a < arg)) {
                    bm = v;
                    arg = a;
                }
            }
            out_arg[p] = arg;
        }
    }
    ll = block_sum_f64(ll, red);
    if (threadIdx.x == 0) part_ll[blockIdx.x] = ll * kLn2;
}

// LL = fixed-order sum of the LL partials; OR of the range flags.  A pass
// that met a value of X outside the fp16 operand range (clamped staging) has
// invalid scores for that point, so its LL is reported as NaN (and the
// finalize that follows keeps theta): the failure is visible in the result.
__global__ __launch_bounds__(256) void k_lk_sum(const double* part_ll, int P, const int* part_flag,
                                                int Pf, double* ll_ws, double* ll_out, int* misc) {
    __shared__ double red[256];
    double v = 0.0;
    for (int p = threadIdx.x; p < P; p += 256) v += part_ll[p];
    v = block_sum_f64(v, red);
    int f = 0;
    for (int p = threadIdx.x; p < Pf; p += 256) f |= part_flag[p];
    f = __syncthreads_or(f);
    if (f) v = __builtin_nan("");
    if (threadIdx.x == 0) {
        *ll_ws = v;
        if (ll_out) *ll_out = v;
        misc[0] = isfinite(v) ? 0 : 1;
        misc[1] = f;
    }
}

// Reduce component k's partials over the point chunks (fixed order), then
// the M-step.  Grid K, 256 threads.  Partial columns are [s0, s1'(D),
// s2'(D)] (diag) or [s0, s1'(D), s2] (iso), with s1' = sum gamma y',
// s2' = sum gamma y'^2, y' = (x - c) s; the isotropic s2 = sum gamma |y|^2.
__global__ __launch_bounds__(256) void k_lk_reduce(
    const double* __restrict__ part, int G, int S, int64_t n, int d, bool iso, float var_floor,
    const float2* __restrict__ dsc, double* __restrict__ stats, float* __restrict__ th_pi,
    float* __restrict__ th_mu, float* __restrict__ th_var, float* __restrict__ out_pi,
    float* __restrict__ out_mu, float* __restrict__ out_var, int* __restrict__ flags,
    const int* __restrict__ misc, const int* __restrict__ xc_pos, const int* __restrict__ xc_n,
    const double* __restrict__ xc_part, int64_t xc_slot_doubles) {
    extern __shared__ double colsum[];   // [ncol]
    __shared__ double red[256];
    const int k = blockIdx.x, tid = threadIdx.x;
    const int ncol = iso ? 2 + d : 1 + 2 * d;
    const int slice = k / kLkSlice, kl = k % kLkSlice;
    const int nchunks = G / S;
    const int pos = xc_pos[k];
    for (int col = tid; col < ncol; col += 256) {
        double a0 = 0.0;
        if (pos < 0) {
            // eight running sums (chunk ch into sum ch % 8), so that eight
            // loads are in flight; combined in a fixed tree
            double a8[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) a8[u] = 0.0;
            int ch = 0;
            for (; ch + 8 <= nchunks; ch += 8) {
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int b = lk_wg_of(slice, ch + u, G, S);
                    a8[u] += part[((int64_t)b * kLkSlice + kl) * ncol + col];
                }
            }
            for (; ch < nchunks; ++ch) {
                const int b = lk_wg_of(slice, ch, G, S);
                a8[ch % 8] += part[((int64_t)b * kLkSlice + kl) * ncol + col];
            }
            a0 = ((a8[0] + a8[1]) + (a8[2] + a8[3])) + ((a8[4] + a8[5]) + (a8[6] + a8[7]));
        } else {   // scored exactly: its own slots (the panel gave it no responsibility)
            const int nx = *xc_n;
            const int P = lk_xc_slots(nx, ncol, xc_slot_doubles, kLkXcSlots);
            for (int b = 0; b < P; ++b) a0 += xc_part[((int64_t)b * nx + pos) * ncol + col];
        }
        colsum[col] = a0;
    }
    __syncthreads();
    const double s0 = colsum[0];
    // a pass with clamped operands (misc[1]) updates nothing: theta is kept
    const bool clamped = misc[1] != 0;
    const bool empty = s0 < kEmptyNk || clamped;
    double nonfin = (isfinite(s0) && !clamped) ? 0.0 : 1.0;
    // per dimension: t1 = sum gamma y, t2 = sum gamma y^2 (diag)
    double mu2 = 0.0, c_t1 = 0.0, cc = 0.0;
    for (int dd = tid; dd < d; dd += 256) {
        const double c = dsc[dd].x, esc = 1.0 / (double)dsc[dd].y;
        const double t1 = colsum[1 + dd] * esc;
        const int64_t i = (int64_t)k * d + dd;
        const int64_t so = (int64_t)k * ncol;
        stats[so + 1 + dd] = t1 + c * s0;
        if (!isfinite(t1)) nonfin = 1.0;
        float mf = th_mu[i];
        if (!empty) mf = (float)(c + t1 / s0);
        const double dm = empty ? 0.0 : t1 / s0;
        if (!iso) {
            const double t2 = colsum[1 + d + dd] * esc * esc;
            stats[so + 1 + d + dd] = t2 + 2.0 * c * t1 + c * c * s0;
            if (!isfinite(t2)) nonfin = 1.0;
            float vf = th_var[i];
            if (!empty) vf = (float)fmax(t2 / s0 - dm * dm, (double)var_floor);
            th_var[i] = vf;
            if (out_var) out_var[i] = vf;
        } else {
            mu2 += dm * dm;
            c_t1 += c * t1;
            cc += c * c;
        }
        th_mu[i] = mf;
        if (out_mu) out_mu[i] = mf;
    }
    nonfin = block_sum_f64(nonfin, red);
    if (iso) {
        mu2 = block_sum_f64(mu2, red);
        c_t1 = block_sum_f64(c_t1, red);
        cc = block_sum_f64(cc, red);
    }
    if (tid == 0) {
        stats[(int64_t)k * ncol] = s0;
        if (iso) {
            const double s2 = colsum[1 + d];
            stats[(int64_t)k * ncol + 1 + d] = s2 + 2.0 * c_t1 + cc * s0;
            if (!isfinite(s2)) nonfin = 1.0;
            float vf = th_var[k];
            if (!empty) vf = (float)fmax((s2 / s0 - mu2) / (double)d, (double)var_floor);
            th_var[k] = vf;
            if (out_var) out_var[k] = vf;
        }
        const float pf = clamped ? th_pi[k] : (float)(s0 / (double)n);
        th_pi[k] = pf;
        if (out_pi) out_pi[k] = pf;
        int f = 0;
        if (!(pf >= 0.0f) || !isfinite(pf)) f |= 1 | 8;
        if (nonfin > 0.0) f |= 8;
        if (empty && !clamped) f |= 4;
        flags[k] = f | (flags[k] & 16);   // keep the conditioning flag of this pass's theta
    }
}

// Centre / scale from a sample of X, then the panel of the current theta.
hipError_t refresh_panel(const Plan& p, const LkWs& w, const void* x, hipStream_t s) {
    const bool iso = p.cov == GMM_COV_ISO;
    if (p.xdt == GMM_BF16)
        hipLaunchKernelGGL(k_lk_scan<true>, dim3(kLkScanWgs), dim3(256), 0, s, (const uint16_t*)x,
                           p.n, p.ldx, (int)p.d, p.dp, w.scan);
    else
        hipLaunchKernelGGL(k_lk_scan<false>, dim3(kLkScanWgs), dim3(256), 0, s, (const uint16_t*)x,
                           p.n, p.ldx, (int)p.d, p.dp, w.scan);
    hipLaunchKernelGGL(k_lk_centre, dim3(1), dim3(1024), 0, s, p.n, (int)p.d, p.dp,
                       p.xdt == GMM_BF16, iso, w.scan, w.dsc, w.prm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_lk_panel<false>, dim3(p.lk_kpad / kKpw), dim3(256), 0, s, (int)p.k, p.lk_kpad,
                       (int)p.d, p.dp, iso, p.lk_kpad / 32, w.pi, w.mu, w.var, w.dsc, w.kmax, w.prm,
                       (uint16_t*)w.panel, w.flags, w.c0, (const int*)w.xc_pos);
    e = lk_xc_build(p, w, s);   // the components flagged above: scored exactly
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_lk_panel<true>, dim3(p.lk_kpad / kKpw), dim3(256), 0, s, (int)p.k, p.lk_kpad,
                       (int)p.d, p.dp, iso, p.lk_kpad / 32, w.pi, w.mu, w.var, w.dsc, w.kmax, w.prm,
                       (uint16_t*)w.panel, w.flags, w.c0, (const int*)w.xc_pos);
    return hipGetLastError();
}

LkArgs make_args(const Plan& p, const LkWs& w, const void* x) {
    LkArgs a;
    memset(&a, 0, sizeof(a));
    a.x = x;
    a.n = p.n;
    a.ldx = p.ldx;
    a.d = (int)p.d;
    a.k_real = (int)p.k;
    a.S = p.lk_slices;
    a.vec = ((uintptr_t)x % 16 == 0 && p.ldx % 8 == 0 && p.d % 8 == 0) ? 1 : 0;
    a.panel = w.panel;
    a.nblk = p.lk_kpad / 32;
    a.prm = w.prm;
    a.dsc = w.dsc;
    a.part = w.part;
    a.part_ll = w.part_ll;
    a.part_flag = w.part_flag;
    a.tlo = 0;
    a.thi = (p.n + kLkT - 1) / kLkT;
    a.seg_first = 1;
    a.xc_n = w.xc_n;
    const size_t rS = (size_t)p.lk_slices * p.n;   // row S: the exactly scored components
    a.xlse = w.part_lse + rS;
    a.xmax = w.part_max + rS;
    a.xarg = w.part_arg + rS;
    a.lse_out = w.part_lse;
    return a;
}

int merge_grid(const Plan& p) {
    int64_t g = (p.n + 255) / 256;
    if (g > kLkMergeWgs) g = kLkMergeWgs;
    return (int)(g < 1 ? 1 : g);
}

// A statistics pass (fused E+M or sweep 2) in segments of at most
// seg_tiles tiles per point chunk: every workgroup's fp32 accumulators are
// closed at the end of each segment and added into its fp64 partial slot.
hipError_t launch_segments(const Plan& p, LkArgs a, int mode, int G, hipStream_t s) {
    const int64_t M = p.seg_tiles > 0 ? p.seg_tiles : kLkSegTiles;
    const LkSegs sg = lk_segs(p.n, G / p.lk_slices, M);
    for (int i = 0; i < sg.n; ++i) {
        a.tlo = (int64_t)i * sg.len;
        a.thi = a.tlo + sg.len < sg.tiles ? a.tlo + sg.len : sg.tiles;
        a.seg_first = i == 0 ? 1 : 0;
        const hipError_t e = lk_launch(p, a, mode, G, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

gmm_status lk_sum(const Plan& p, const LkWs& w, int P, int Pf, double* ll_out, hipStream_t s) {
    hipLaunchKernelGGL(k_lk_sum, dim3(1), dim3(256), 0, s, w.part_ll, P, w.part_flag, Pf, w.ll,
                       ll_out, w.misc);
    return hipGetLastError() == hipSuccess ? GMM_OK : GMM_E_HIP;
}

}  // namespace

// Grid: lk_wg_per_cu(mode) workgroups per CU, chunks a multiple of 8 so that
// each chunk's slices share an XCD; never more chunks than tiles, partial
// slots (statistics modes) or LL / flag slots.
int lk_grid(const Plan& p, int mode) {
    const int mb = lk_plan_mode(p, mode);
    // workgroups per point chunk (top-m: one slice per launch)
    const int S = mode == LK_TOPM ? 1 : p.lk_slices / lk_slices_per_wg(mb);
    const int64_t tiles = (p.n + kLkT - 1) / kLkT;
    int64_t chunks = (int64_t)lk_wg_per_cu(mb) * device_cu_count() / S;
    if (chunks >= 8) chunks = chunks / 8 * 8;
    if (chunks < 1) chunks = 1;
    if (chunks > tiles) chunks = tiles < 1 ? 1 : tiles;
    const bool stats = mode == LK_FUSED_EM || mode == LK_SWEEP2;
    const int64_t slots = stats ? p.p_max : kLkLLSlots;
    if (chunks * S > slots) chunks = slots / S;
    return (int)(chunks * S);
}

gmm_status lk_prepare(const Plan& p, char* ws, const float* pi, const float* mu, const float* var,
                      hipStream_t s) {
    LkWs w = lk_ws(p, ws);
    hipLaunchKernelGGL(k_lk_load, dim3(p.k), dim3(128), 0, s, (int)p.k, (int)p.d,
                       p.cov == GMM_COV_ISO, pi, mu, var, w.pi, w.mu, w.var, w.flags, w.xc_pos, w.xc_n);
    return hipGetLastError() == hipSuccess ? GMM_OK : GMM_E_HIP;
}

gmm_status lk_em_step(const Plan& p, char* ws, const void* x, double* ll_out, hipStream_t s) {
    LkWs w = lk_ws(p, ws);
    if (refresh_panel(p, w, x, s) != hipSuccess) return GMM_E_HIP;
    LkArgs a = make_args(p, w, x);
    if (p.lk_slices == 1) {
        const int G = lk_grid(p, LK_FUSED_EM);
        if (lk_xc_lse(p, w, x, s) != hipSuccess) return GMM_E_HIP;
        if (launch_segments(p, a, LK_FUSED_EM, G, s) != hipSuccess) return GMM_E_HIP;
        if (lk_xc_stats(p, w, x, s) != hipSuccess) return GMM_E_HIP;
        return lk_sum(p, w, G, G, ll_out, s);
    }
    const int G1 = lk_grid(p, LK_SWEEP1), G = lk_grid(p, LK_SWEEP2);
    a.part_lse = w.part_lse;
    if (lk_launch(p, a, LK_SWEEP1, G1, s) != hipSuccess) return GMM_E_HIP;
    if (lk_xc_lse(p, w, x, s) != hipSuccess) return GMM_E_HIP;
    const int M = merge_grid(p);
    hipLaunchKernelGGL(k_lk_merge, dim3(M), dim3(256), 0, s, p.n, p.lk_slices, w.part_lse,
                       (const int*)nullptr, (const float*)nullptr, w.part_ll, (float*)nullptr,
                       (int*)nullptr, (const int*)w.xc_n);
    if (hipGetLastError() != hipSuccess) return GMM_E_HIP;
    a.part_lse = nullptr;
    a.lse_in = w.part_lse;
    if (launch_segments(p, a, LK_SWEEP2, G, s) != hipSuccess) return GMM_E_HIP;
    if (lk_xc_stats(p, w, x, s) != hipSuccess) return GMM_E_HIP;
    // range flags: sweep 1 wrote slots [0, G1), sweep 2 rewrote [0, G)
    return lk_sum(p, w, M, G1 > G ? G1 : G, ll_out, s);
}

gmm_status lk_finalize(const Plan& p, char* ws, float* pi, float* mu, float* var, hipStream_t s) {
    LkWs w = lk_ws(p, ws);
    const int G = lk_grid(p, p.lk_slices == 1 ? LK_FUSED_EM : LK_SWEEP2);
    const size_t shm = sizeof(double) * (size_t)p.ncols;
    hipLaunchKernelGGL(k_lk_reduce, dim3(p.k), dim3(256), shm, s, w.part, G, p.lk_slices, p.n,
                       (int)p.d, p.cov == GMM_COV_ISO, p.var_floor, w.dsc, w.stats, w.pi, w.mu,
                       w.var, pi, mu, var, w.flags, w.misc, (const int*)w.xc_pos, (const int*)w.xc_n,
                       (const double*)w.xc_part, w.xc_slot_doubles);
    return hipGetLastError() == hipSuccess ? GMM_OK : GMM_E_HIP;
}

// Top-m assignment: sweep 1 and the slice merge give every point's LSE, then
// one top-m launch per slice, each merging its slice's candidates into the
// running list (the outputs) in slice order.
gmm_status lk_assign(const Plan& p, char* ws, const void* x, int m, int32_t* idx, float* gamma,
                     double* ll_out, hipStream_t s) {
    LkWs w = lk_ws(p, ws);
    if (p.n == 0) return lk_sum(p, w, 0, 0, ll_out, s);
    if (refresh_panel(p, w, x, s) != hipSuccess) return GMM_E_HIP;
    LkArgs a = make_args(p, w, x);
    const int G1 = lk_grid(p, LK_SWEEP1);
    a.part_lse = w.part_lse;
    if (lk_launch(p, a, LK_SWEEP1, G1, s) != hipSuccess) return GMM_E_HIP;
    if (lk_xc_lse(p, w, x, s) != hipSuccess) return GMM_E_HIP;
    const int M = merge_grid(p);
    hipLaunchKernelGGL(k_lk_merge, dim3(M), dim3(256), 0, s, p.n, p.lk_slices, w.part_lse,
                       (const int*)nullptr, (const float*)nullptr, w.part_ll, (float*)nullptr,
                       (int*)nullptr, (const int*)w.xc_n);
    if (hipGetLastError() != hipSuccess) return GMM_E_HIP;
    a.part_lse = nullptr;
    a.lse_in = w.part_lse;
    a.topm = m;
    a.out_idx = idx;
    a.out_gamma = gamma;
    // the exactly scored components start every point's running list
    if (lk_xc_topm(p, w, x, m, idx, gamma, s) != hipSuccess) return GMM_E_HIP;
    const int GT = lk_grid(p, LK_TOPM);
    for (int sl = 0; sl < p.lk_slices; ++sl) {
        a.topm_slice = sl;
        if (lk_launch(p, a, LK_TOPM, GT, s) != hipSuccess) return GMM_E_HIP;
    }
    return lk_sum(p, w, M, G1 > GT ? G1 : GT, ll_out, s);
}

gmm_status lk_loglik(const Plan& p, char* ws, const void* x, double* ll_out, float* lse,
                     int32_t* argmax, hipStream_t s) {
    LkWs w = lk_ws(p, ws);
    if (p.n == 0) return lk_sum(p, w, 0, 0, ll_out, s);
    if (refresh_panel(p, w, x, s) != hipSuccess) return GMM_E_HIP;
    const int G = lk_grid(p, p.lk_slices == 1 ? LK_FUSED_E : LK_SWEEP1);
    LkArgs a = make_args(p, w, x);
    if (p.lk_slices == 1) {
        a.out_lse = lse;
        a.out_arg = argmax;
        if (lk_xc_lse(p, w, x, s) != hipSuccess) return GMM_E_HIP;
        if (lk_launch(p, a, LK_FUSED_E, G, s) != hipSuccess) return GMM_E_HIP;
        return lk_sum(p, w, G, G, ll_out, s);
    }
    a.part_lse = w.part_lse;
    if (argmax) {
        a.part_arg = w.part_arg;
        a.part_max = w.part_max;
    }
    if (lk_launch(p, a, LK_SWEEP1, G, s) != hipSuccess) return GMM_E_HIP;
    if (lk_xc_lse(p, w, x, s) != hipSuccess) return GMM_E_HIP;
    const int M = merge_grid(p);
    hipLaunchKernelGGL(k_lk_merge, dim3(M), dim3(256), 0, s, p.n, p.lk_slices, w.part_lse,
                       (const int*)w.part_arg, (const float*)w.part_max, w.part_ll, lse, argmax,
                       (const int*)w.xc_n);
    if (hipGetLastError() != hipSuccess) return GMM_E_HIP;
    return lk_sum(p, w, M, G, ll_out, s);
}

}  // namespace gmm
