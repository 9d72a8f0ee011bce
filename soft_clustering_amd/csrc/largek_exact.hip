// Large-K family: the components scored in the exact centred form.
//
// The fp16 expanded-form score [y'^2 | y' | bias] . panel cannot resolve a
// component whose variance is small against its distance from the centre
// (say one that collapsed onto a few points): the terms A y'^2 and B y'
// cancel to a result far below their rounding error.  The panel preparation
// flags such components (flag bit 4: estimated error near their own mean above
// a few nats); they are taken out of the fp16 panel (score -inf there) and
// scored here directly, d^2 = sum_d (x_d - mu_d)^2 / var_d in fp32 from the
// stored x ([LP-GMM] 1.2 density; 1.3, the precision of exp / log /
// denominators / statistics stays fp32 or wider):
//
//   k_xc_build  - the list of flagged components in index order;
//   k_xc_lse    - per point their base-2 log-sum-exp, largest score and its
//                 component: one more row next to the 256-component slices'
//                 LSE, merged with them (or, with one slice, inside the fused
//                 kernel) into every point's normaliser;
//   k_xc_stats  - their responsibilities exp2(S - lse) against the merged LSE
//                 and s0 / s1 / s2 in the fused kernel's units, fp32 over
//                 256-point tiles and fp64 across tiles, in workgroup slots
//                 of their own that the reduction adds to the others;
//   k_xc_topm   - their top-m lists per point, the start of the running lists
//                 that the slices' top-m passes merge into.
// Every kernel reads the count first and returns at once when no component is
// flagged, so a pass without ill-conditioned components costs a few empty
// launches.

#include <type_traits>

#include "largek_internal.h"

namespace gmm {

namespace {

constexpr float kHalfLog2eF = 0.72134752044448170368f;

template <bool BF16>
__device__ __forceinline__ float h16(uint32_t bits16) {
    if constexpr (BF16) return __uint_as_float(bits16 << 16);
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// Row p of X as fp32 in xv[0, DP) (zero beyond D).
template <int DP, bool BF16, bool VEC>
__device__ __forceinline__ void load_row(const uint16_t* __restrict__ x, int64_t p, int64_t ldx, int d,
                                         float (&xv)[DP]) {
    const uint16_t* row = x + p * ldx;
    if constexpr (VEC) {
#pragma unroll
        for (int c = 0; c < DP / 8; ++c) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (8 * c < d) v = *reinterpret_cast<const uint4*>(row + 8 * c);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                xv[8 * c + 2 * q] = 8 * c < d ? h16<BF16>(w[q] & 0xFFFFu) : 0.0f;
                xv[8 * c + 2 * q + 1] = 8 * c < d ? h16<BF16>(w[q] >> 16) : 0.0f;
            }
        }
    } else {
#pragma unroll
        for (int dd = 0; dd < DP; ++dd) xv[dd] = dd < d ? h16<BF16>(row[dd]) : 0.0f;
    }
}

// Base-2 centred-form score of component k at xv.
template <int DP>
__device__ __forceinline__ float exact_score(const float (&xv)[DP], int d, bool iso, int k,
                                             const float* __restrict__ mu, const float* __restrict__ var,
                                             const float* __restrict__ c0) {
    const float ck = c0[k];
    if (ck == -INFINITY) return -INFINITY;
    float q = 0.0f;
    const float* mk = mu + (int64_t)k * d;
    if (iso) {
#pragma unroll
        for (int dd = 0; dd < DP; ++dd) {
            if (dd < d) {
                const float df = xv[dd] - mk[dd];
                q = fmaf(df, df, q);
            }
        }
        q = q / var[k];
    } else {
        const float* vk = var + (int64_t)k * d;
#pragma unroll
        for (int dd = 0; dd < DP; ++dd) {
            if (dd < d) {
                const float df = xv[dd] - mk[dd];
                q = fmaf(df * df, 1.0f / vk[dd], q);
            }
        }
    }
    return ck - kHalfLog2eF * q;
}

// The flagged components in index order; position of every component in the
// list (-1: scored by the panel).  One workgroup of 256 threads, each taking
// a contiguous run of components.
__global__ __launch_bounds__(256) void k_xc_build(int k_real, const int* __restrict__ flags,
                                                  int* __restrict__ xc_idx, int* __restrict__ xc_pos,
                                                  int* __restrict__ xc_n) {
    __shared__ int cnt[256];
    const int t = threadIdx.x;
    const int per = (k_real + 255) / 256;
    const int k0 = t * per, k1 = k0 + per < k_real ? k0 + per : k_real;
    int c = 0;
    for (int k = k0; k < k1; ++k) c += (flags[k] & 16) ? 1 : 0;
    cnt[t] = c;
    __syncthreads();
    if (t == 0) {
        int s = 0;
        for (int i = 0; i < 256; ++i) {
            const int v = cnt[i];
            cnt[i] = s;
            s += v;
        }
        *xc_n = s;
    }
    __syncthreads();
    int pos = cnt[t];
    for (int k = k0; k < k1; ++k) {
        if (flags[k] & 16) {
            xc_idx[pos] = k;
            xc_pos[k] = pos++;
        } else {
            xc_pos[k] = -1;
        }
    }
}

// Per point: base-2 LSE over the listed components, the largest score and
// its component (lowest index on ties).  Grid-stride over points.
template <int DP, bool BF16, bool VEC>
__global__ __launch_bounds__(256) void k_xc_lse(const uint16_t* __restrict__ x, int64_t n, int64_t ldx,
                                                int d, int iso, const float* __restrict__ mu,
                                                const float* __restrict__ var, const float* __restrict__ c0,
                                                const int* __restrict__ xc_idx, const int* __restrict__ xc_n,
                                                float* __restrict__ xlse, float* __restrict__ xmax,
                                                int* __restrict__ xarg) {
    const int nx = *xc_n;
    if (nx == 0) return;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x; p < n; p += stride) {
        float xv[DP];
        load_row<DP, BF16, VEC>(x, p, ldx, d, xv);
        float M = -INFINITY, Z = 0.0f;
        int arg = -1;
        for (int j = 0; j < nx; ++j) {
            const int k = xc_idx[j];
            const float s = exact_score<DP>(xv, d, iso != 0, k, mu, var, c0);
            if (s == -INFINITY) continue;
            if (s > M) {
                Z = Z * fast_exp2(M - s) + 1.0f;
                M = s;
                arg = k;
            } else {
                Z += fast_exp2(s - M);
            }
        }
        xlse[p] = M == -INFINITY ? -INFINITY : M + fast_log2(Z);
        xmax[p] = M;
        xarg[p] = arg < 0 ? 0x7FFFFFFF : arg;
    }
}

// Statistics of the listed components.  Workgroup b < P (as many slots of
// nx x ncol doubles as the slot area holds, at most the grid) takes a
// contiguous range of points; per chunk of 16 listed components, 256-point
// tiles: each thread stages one point (raw storage bits) and its 16
// responsibilities, then thread (j, q) sums component j's columns for
// dimensions q, q + 16, ... over the tile in fp32 and adds the tile into fp64.
// Columns as the fused kernel's partials: diag [s0, sum g y', sum g y'^2],
// iso [s0, sum g y', sum g |x - c|^2], y' = (x - c) s.
template <int DP, bool BF16, bool VEC>
__global__ __launch_bounds__(256) void k_xc_stats(const uint16_t* __restrict__ x, int64_t n, int64_t ldx,
                                                  int d, int iso, const float* __restrict__ mu,
                                                  const float* __restrict__ var, const float* __restrict__ c0,
                                                  const float2* __restrict__ dsc, const int* __restrict__ xc_idx,
                                                  const int* __restrict__ xc_n, const float* __restrict__ lse,
                                                  double* __restrict__ xc_part, int64_t slot_doubles, int ncol) {
    constexpr int ND = DP / 16;
    __shared__ uint16_t xt[256][DP + 2];
    __shared__ float gt[16][256];
    __shared__ float2 cs[DP];
    const int nx = *xc_n;
    if (nx == 0) return;
    const int P = lk_xc_slots(nx, ncol, slot_doubles, gridDim.x);
    const int b = blockIdx.x;
    if (b >= P) return;
    const int t = threadIdx.x, jl = t >> 4, q = t & 15;
    for (int i = t; i < DP; i += 256) cs[i] = i < d ? dsc[i] : make_float2(0.0f, 0.0f);
    const int64_t per = (n + P - 1) / P;
    const int64_t p0 = (int64_t)b * per, p1 = p0 + per < n ? p0 + per : n;
    for (int cj = 0; cj < nx; cj += 16) {
        const int nj = nx - cj < 16 ? nx - cj : 16;
        double a0 = 0.0, a1[ND], a2[ND];
#pragma unroll
        for (int i = 0; i < ND; ++i) a1[i] = a2[i] = 0.0;
        for (int64_t pt = p0; pt < p1; pt += 256) {
            const int64_t pp = pt + t;
            const bool valid = pp < p1;
            float xv[DP];
            load_row<DP, BF16, VEC>(x, valid ? pp : p0, ldx, d, xv);
#pragma unroll
            for (int dd = 0; dd < DP; ++dd) {
                uint16_t bits;
                if constexpr (BF16) bits = (uint16_t)(__float_as_uint(xv[dd]) >> 16);
                else bits = __builtin_bit_cast(uint16_t, (_Float16)xv[dd]);
                xt[t][dd] = bits;
            }
            const float l = valid ? lse[pp] : INFINITY;
            for (int j = 0; j < nj; ++j) {
                const float s = exact_score<DP>(xv, d, iso != 0, xc_idx[cj + j], mu, var, c0);
                gt[j][t] = valid ? fast_exp2(s - l) : 0.0f;
            }
            __syncthreads();
            if (jl < nj) {
                float s0 = 0.0f, s1[ND], s2[ND];
#pragma unroll
                for (int i = 0; i < ND; ++i) s1[i] = s2[i] = 0.0f;
                for (int i = 0; i < 256; ++i) {
                    const float g = gt[jl][i];
                    if (g == 0.0f) continue;
                    s0 += g;
#pragma unroll
                    for (int di = 0; di < ND; ++di) {
                        const int dd = q + 16 * di;
                        const float2 c = cs[dd];
                        const float xd = h16<BF16>(xt[i][dd]) - c.x;
                        const float y = iso ? xd : xd * c.y;
                        s1[di] = fmaf(g, iso ? xd * c.y : y, s1[di]);
                        s2[di] = fmaf(g, y * y, s2[di]);
                    }
                }
                a0 += (double)s0;
#pragma unroll
                for (int i = 0; i < ND; ++i) {
                    a1[i] += (double)s1[i];
                    a2[i] += (double)s2[i];
                }
            }
            __syncthreads();
        }
        if (jl < nj) {
            double* dst = xc_part + ((int64_t)b * nx + cj + jl) * ncol;
            if (q == 0) dst[0] = a0;
            double sq = 0.0;
#pragma unroll
            for (int di = 0; di < ND; ++di) {
                const int dd = q + 16 * di;
                if (dd < d) {
                    dst[1 + dd] = a1[di];
                    if (!iso) dst[1 + d + dd] = a2[di];
                    else sq += a2[di];
                }
            }
            if (iso) {   // sum over the dimensions: the 16 lanes of this component, fixed tree
#pragma unroll
                for (int o = 8; o > 0; o >>= 1) sq += __shfl_xor(sq, o, 16);
                if (q == 0) dst[1 + d] = sq;
            }
        }
    }
}

// Top-m of the listed components per point (base-2 scores; lowest index
// first on ties): the start of the running lists.
template <int DP, bool BF16, bool VEC>
__global__ __launch_bounds__(256) void k_xc_topm(const uint16_t* __restrict__ x, int64_t n, int64_t ldx,
                                                 int d, int iso, const float* __restrict__ mu,
                                                 const float* __restrict__ var, const float* __restrict__ c0,
                                                 const int* __restrict__ xc_idx, const int* __restrict__ xc_n,
                                                 int m, int* __restrict__ out_idx, float* __restrict__ out_score) {
    const int nx = *xc_n;
    if (nx == 0) return;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x; p < n; p += stride) {
        float xv[DP];
        load_row<DP, BF16, VEC>(x, p, ldx, d, xv);
        float tv[kLkMaxTopm];
        int ti[kLkMaxTopm];
#pragma unroll
        for (int i = 0; i < kLkMaxTopm; ++i) {
            tv[i] = -INFINITY;
            ti[i] = -1;
        }
        for (int j = 0; j < nx; ++j) {
            const int k = xc_idx[j];
            float v = exact_score<DP>(xv, d, iso != 0, k, mu, var, c0);
            if (v == -INFINITY) continue;
            int kk = k;
            // insertion into the sorted list (strictly larger moves ahead, so an
            // equal score keeps the lower, earlier index in front)
#pragma unroll
            for (int i = 0; i < kLkMaxTopm; ++i) {
                if (i < m && (ti[i] < 0 || v > tv[i])) {
                    const float tv0 = tv[i];
                    const int ti0 = ti[i];
                    tv[i] = v;
                    ti[i] = kk;
                    v = tv0;
                    kk = ti0;
                    if (kk < 0) break;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < kLkMaxTopm; ++i) {
            if (i < m) {
                out_idx[p * m + i] = ti[i];
                out_score[p * m + i] = ti[i] < 0 ? 0.0f : tv[i];
            }
        }
    }
}

int xc_grid(const Plan& p) {
    int64_t g = (p.n + 255) / 256;
    const int64_t cap = 4 * (int64_t)device_cu_count();
    if (g > cap) g = cap;
    return (int)(g < 1 ? 1 : g);
}

bool xc_vec(const Plan& p, const void* x) {
    return (uintptr_t)x % 16 == 0 && p.ldx % 8 == 0 && p.d % 8 == 0;
}

}  // namespace

hipError_t lk_xc_build(const Plan& p, const LkWs& w, hipStream_t s) {
    hipLaunchKernelGGL(k_xc_build, dim3(1), dim3(256), 0, s, (int)p.k, (const int*)w.flags, w.xc_idx,
                       w.xc_pos, w.xc_n);
    return hipGetLastError();
}

#define XC_DISPATCH(KERNEL, GRID, ...)                                                              \
    do {                                                                                            \
        const bool bf = p.xdt == GMM_BF16, vec = xc_vec(p, x);                                      \
        auto go = [&](auto dpc, auto bfc, auto vc) {                                                \
            hipLaunchKernelGGL((KERNEL<decltype(dpc)::value, decltype(bfc)::value, decltype(vc)::value>), \
                               dim3(GRID), dim3(256), 0, s, __VA_ARGS__);                           \
        };                                                                                          \
        auto go2 = [&](auto dpc) {                                                                  \
            if (bf && vec) go(dpc, std::true_type{}, std::true_type{});                             \
            else if (bf) go(dpc, std::true_type{}, std::false_type{});                              \
            else if (vec) go(dpc, std::false_type{}, std::true_type{});                             \
            else go(dpc, std::false_type{}, std::false_type{});                                     \
        };                                                                                          \
        if (p.dp == 32) go2(std::integral_constant<int, 32>{});                                     \
        else if (p.dp == 64) go2(std::integral_constant<int, 64>{});                                \
        else go2(std::integral_constant<int, 128>{});                                               \
    } while (0)

hipError_t lk_xc_lse(const Plan& p, const LkWs& w, const void* x, hipStream_t s) {
    const int S = p.lk_slices;
    XC_DISPATCH(k_xc_lse, xc_grid(p), (const uint16_t*)x, p.n, p.ldx, (int)p.d,
                p.cov == GMM_COV_ISO ? 1 : 0, (const float*)w.mu, (const float*)w.var, (const float*)w.c0,
                (const int*)w.xc_idx, (const int*)w.xc_n, w.part_lse + (size_t)S * p.n,
                w.part_max + (size_t)S * p.n, w.part_arg + (size_t)S * p.n);
    return hipGetLastError();
}

hipError_t lk_xc_stats(const Plan& p, const LkWs& w, const void* x, hipStream_t s) {
    XC_DISPATCH(k_xc_stats, kLkXcSlots, (const uint16_t*)x, p.n, p.ldx, (int)p.d,
                p.cov == GMM_COV_ISO ? 1 : 0, (const float*)w.mu, (const float*)w.var, (const float*)w.c0,
                (const float2*)w.dsc, (const int*)w.xc_idx, (const int*)w.xc_n, (const float*)w.part_lse,
                w.xc_part, w.xc_slot_doubles, (int)p.ncols);
    return hipGetLastError();
}

hipError_t lk_xc_topm(const Plan& p, const LkWs& w, const void* x, int m, int* idx, float* score,
                      hipStream_t s) {
    XC_DISPATCH(k_xc_topm, xc_grid(p), (const uint16_t*)x, p.n, p.ldx, (int)p.d,
                p.cov == GMM_COV_ISO ? 1 : 0, (const float*)w.mu, (const float*)w.var, (const float*)w.c0,
                (const int*)w.xc_idx, (const int*)w.xc_n, m, idx, score);
    return hipGetLastError();
}

}  // namespace gmm
