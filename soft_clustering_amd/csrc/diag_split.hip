// Fused E-step + M-step statistics for a diagonal-covariance GMM, fp32
// accuracy on the fp16 matrix cores.
//
// Method: [Flash-GMM] Method, fused E-M step (tile X along N; per tile the
// Mahalanobis terms and the softmax over all K stay on chip; s0/s1/s2 are
// accumulated in the same pass, the N x K responsibilities never reach HBM).
// Density and posterior: [LP-GMM] 1.1-1.2; log-space posterior with max
// shift: [LP-GMM] 4.2.  Precision boundaries: matrix products may run on
// fp16 operands while exp, log, denominators and statistic accumulation stay
// in fp32 or wider, and fp16 operands must be kept inside the fp16 range
// ([LP-GMM] 1.3, 2.1).
//
// Score as a contraction.  For a diagonal covariance
//   log2(pi_k N(x | mu_k, sigma_k^2)) = sum_d a_kd y_d^2 + b_kd y_d + c_k,
// with y = (x - c) s (per-dimension centre c and power-of-two scale s) and
// a_kd, b_kd the precision terms in those units, so a 16-point x
// 16-component score block is [y^2 | y] (16 x 2D) times the panel [a ; b]
// (2D x 16 per component block, divided by a per-component power of two F_k).
//
// Split fp16.  Every operand v of both contractions is carried as
// hi + lo, hi = fp16(v), lo = fp16(v - hi) (22 significant bits), and each
// product as hi*hi + hi*lo + lo*hi on v_mfma_f32_16x16x32_f16 with fp32
// accumulation; the dropped lo*lo term is below 2^-22 of the product.  The
// result carries the rounding of an fp32 contraction to within a small
// factor, at the fp16 MFMA rate (three fp16 products cost less than one
// v_mfma_f32_16x16x4f32 of the same size).  The scale s keeps a tile's y
// well inside the fp16 range; a tile with any |y| above kSplitLim (an
// outlier far outside the model's spread) is computed instead with fp32
// MFMAs on operands read back from global memory, so no input changes the
// result beyond fp32 rounding.
//
// Layout.  A wave owns a contiguous run of 32-point tiles.  Each tile is
// loaded global -> registers (the loads of tile t+1 are issued as soon as
// tile t has been staged, and land while it is computed), split into a wave-private LDS tile pair H / L [point][2D]
// (columns: y^2 then y), and consumed twice: the score MFMA reads rows of
// H / L as its A operand (points x features), the statistics MFMA reads
// columns with ds_read_b64_tr_b16 as its B operand (points as K).  The score
// accumulator of a 16-point group (lane (g, j): points 4g+r of component j)
// is, after the softmax and the split, exactly the A operand (components x
// points) of the statistics product, so responsibilities never leave
// registers.  16-byte units of a tile row are XOR-swizzled by the row so
// that both access patterns hit 16 distinct units per LDS cycle.
//
// Each workgroup writes one fp64 partial of (s0, S1, S2) and of LL (moments
// of y about c); later kernels sum them in a fixed order and undo the scale.
// This translation unit is compiled with IEEE mode off and no-NaN
// assumptions (the DPP max folds into v_max_f32_dpp); non-finite results are
// detected by the kernels that consume the partials.

#include "diag_internal.h"

namespace gmm {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

constexpr int kST = 32;   // points per tile

template <int DP, int KB, typename XT>
struct SplitShape {
    static constexpr int kWaves = diag_split_waves(DP, KB);
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kKS = DP / 16;              // score k-steps of 32 (contraction 2 DP)
    static constexpr int kNCB = DP / 8;              // statistic column blocks of 16 (2 DP columns)
    static constexpr int kPitch = DP <= 64 ? 128 : 2 * DP;   // halves per tile row (>= 256 B)
    static constexpr int kTile = kST * kPitch;       // halves per tile array
    static constexpr int kEV = Vec16<XT>::kElems;    // elements per 16-byte vector
    static constexpr int kVPR = DP / kEV;            // vectors per row
    static constexpr int kPer = kST * kVPR / 64;     // vectors per lane per tile
    static_assert(kPer >= 1 && 64 % kVPR == 0, "tile geometry");
};

// XOR swizzle of the 16-byte units of tile row r.  Rows 0..15 map to 16
// distinct values (row reads of 16 points hit 16 units), and rows r, r+1,
// ..., r+7 with r % 8 == 0 map to 8 distinct unit pairs (the 32-byte
// column reads of ds_read_b64_tr_b16).
__device__ __forceinline__ int swz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

template <int PITCH>
__device__ __forceinline__ int uoff(int r, int u) { return r * PITCH + ((u ^ swz(r)) << 3); }

// Tile row loaded by vector slot t (0..31): consecutive lane groups of a load
// get rows that differ in bit 2, whose swizzles cover complementary halves
// of a 256-byte row, so the staging writes of one LDS cycle do not collide.
__device__ __forceinline__ int row_of(int t) { return (t & 24) | ((t & 1) << 2) | ((t >> 1) & 3); }

// ds_read_b64_tr_b16: in each group of 16 lanes, lane i' reads 4 halves of
// row (i' / 4) at column 4 (i' % 4) (addresses as given); lane i receives
// column i of the 4 rows.
__device__ __forceinline__ uint2 tr16(const uint16_t* p) {
    const short4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)((lds_u16*)p));
    return __builtin_bit_cast(uint2, v);
}

// A wave-uniform 64-bit value, moved to scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ f32x4 mfma_f16(const half8& a, const half8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Order this wave's LDS writes before its later LDS reads and the reads
// before later writes (one wave: a compiler / memory fence at wavefront
// scope, no s_barrier).
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Global -> register loads of one 32-point tile.  Vector slot i of a lane
// reads row row_of((lane + 64 i) / kVPR) at column (lane % kVPR) kEV
// (column 0 when that lies past D: the scale of such columns is zero, so
// they stage as zero; a non-finite value there makes its row's scores
// non-finite anyway).  The byte offsets of these (row, column) pairs are
// fixed per lane, so a tile is read from one uniform base.  A problem of
// fewer than 32 points clamps its rows to the last one.  On the
// element-wise path columns beyond D read as zero.  Nothing is masked after
// the load (that would make the compiler wait for it).
template <typename XT, int DP, int KB, bool VEC>
struct TileRegs {
    using S = SplitShape<DP, KB, XT>;
    uint4 raw[S::kPer];

    __device__ __forceinline__ void load(const XT* __restrict__ xt, const uint32_t (&off)[S::kPer],
                                         int d, int lane) {
        if constexpr (VEC) {
            // an opaque scalar base and 32-bit offsets: keeps the compiler from
            // folding them into loop-invariant 64-bit vector addresses (the
            // scalar-base form needs no address registers or adds)
            typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
            typedef __attribute__((address_space(1))) const char gchar;
            typedef __attribute__((address_space(1))) const u32x4 gu32x4;
            gchar* base = (gchar*)xt;
            asm volatile("" : "+s"(base));
#pragma unroll
            for (int i = 0; i < S::kPer; ++i) {
                uint32_t o = off[i];
                asm volatile("" : "+v"(o));
                const u32x4 v = *(gu32x4*)(base + o);
                raw[i] = make_uint4(v.x, v.y, v.z, v.w);
            }
        } else {
            // off[i]: element offset of the row; the lane's columns are fixed
            const int col0 = (lane % S::kVPR) * S::kEV;
#pragma unroll
            for (int i = 0; i < S::kPer; ++i) {
                const XT* __restrict__ row = xt + off[i];
                uint32_t w[4];
                if constexpr (S::kEV == 4) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        w[e] = col0 + e < d ? __float_as_uint(to_f32(row[col0 + e])) : 0u;
                } else {
                    const uint16_t* rb = reinterpret_cast<const uint16_t*>(row);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t lo = col0 + 2 * e < d ? rb[col0 + 2 * e] : 0u;
                        const uint32_t hi = col0 + 2 * e + 1 < d ? rb[col0 + 2 * e + 1] : 0u;
                        w[e] = lo | (hi << 16);
                    }
                }
                raw[i] = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
    }
};

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));

// hi = fp16(v) (round to nearest even, both lanes in one conversion) and
// lo = fp16(v - hi): v - hi is exact in fp32 and rounded once, by one
// mixed-precision fma per value that reads hi as fp16 and writes its fp16
// result into one half of the packed register.
__device__ __forceinline__ void split2(float v0, float v1, uint32_t& hi, uint32_t& lo) {
    const half2v h = __builtin_convertvector((float2v){v0, v1}, half2v);
    hi = __builtin_bit_cast(uint32_t, h);
    uint32_t l;
    asm("v_fma_mixlo_f16 %0, %1, 1.0, -%2 op_sel_hi:[0,0,1]" : "=v"(l) : "v"(v0), "v"(hi));
    asm("v_fma_mixhi_f16 %0, %1, 1.0, -%2 op_sel:[0,0,1] op_sel_hi:[0,0,1]" : "+v"(l) : "v"(v1), "v"(hi));
    lo = l;
}

// y^2 from the split of y (h + l, packed pairs): h2 = fp16(h h), the
// remainder h h - h2 (exact in fp16) plus 2 h l rounded once as the low
// part; the dropped l^2 and that rounding are below 2^-21 of y^2.
__device__ __forceinline__ void square2(uint32_t hi, uint32_t lo, uint32_t& hi2, uint32_t& lo2) {
    const half2v h = __builtin_bit_cast(half2v, hi), l = __builtin_bit_cast(half2v, lo);
    const half2v h2 = h * h;
    const half2v ex = __builtin_elementwise_fma(h, h, -h2);
    hi2 = __builtin_bit_cast(uint32_t, h2);
    lo2 = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(h + h, l, ex));
}

// Split a tile into H / L (columns [y^2 | y]); returns this lane's max |y|.
template <typename XT, int DP, int KB>
__device__ __forceinline__ float stage_tile(const uint4 (&raw)[SplitShape<DP, KB, XT>::kPer],
                                            uint16_t* __restrict__ H, uint16_t* __restrict__ L,
                                            const float (&sv)[SplitShape<DP, KB, XT>::kEV],
                                            const float (&csv)[SplitShape<DP, KB, XT>::kEV],
                                            int lane) {
    using S = SplitShape<DP, KB, XT>;
    constexpr int EV = S::kEV;
    const int col0 = (lane % S::kVPR) * EV;
    float mx = 0.0f;
#pragma unroll
    for (int i = 0; i < S::kPer; ++i) {
        const int r = row_of((lane + 64 * i) / S::kVPR);
        float xv[EV];
        Vec16<XT>::unpack(raw[i], xv);
        uint32_t h1[EV / 2], l1[EV / 2], h2[EV / 2], l2[EV / 2];
#pragma unroll
        for (int e = 0; e < EV; e += 2) {
            // (x - c) s in one rounding (c s is exact: s is a power of two)
            const float y0 = fmaf(xv[e], sv[e], -csv[e]);
            const float y1 = fmaf(xv[e + 1], sv[e + 1], -csv[e + 1]);
            mx = fmaxf(mx, fmaxf(fabsf(y0), fabsf(y1)));
            split2(y0, y1, h1[e / 2], l1[e / 2]);
            square2(h1[e / 2], l1[e / 2], h2[e / 2], l2[e / 2]);
        }
        // y^2 at columns [0, DP), y at [DP, 2 DP)
        const int o2 = uoff<S::kPitch>(r, col0 / 8) + (col0 & 7);
        const int o1 = uoff<S::kPitch>(r, (DP + col0) / 8) + (col0 & 7);
        if constexpr (EV == 8) {
            *reinterpret_cast<uint4*>(H + o2) = make_uint4(h2[0], h2[1], h2[2], h2[3]);
            *reinterpret_cast<uint4*>(L + o2) = make_uint4(l2[0], l2[1], l2[2], l2[3]);
            *reinterpret_cast<uint4*>(H + o1) = make_uint4(h1[0], h1[1], h1[2], h1[3]);
            *reinterpret_cast<uint4*>(L + o1) = make_uint4(l1[0], l1[1], l1[2], l1[3]);
        } else {
            *reinterpret_cast<uint2*>(H + o2) = make_uint2(h2[0], h2[1]);
            *reinterpret_cast<uint2*>(L + o2) = make_uint2(l2[0], l2[1]);
            *reinterpret_cast<uint2*>(H + o1) = make_uint2(h1[0], h1[1]);
            *reinterpret_cast<uint2*>(L + o1) = make_uint2(l1[0], l1[1]);
        }
    }
    return mx;
}

// y of point p, dimension dd (fp32; zero beyond D), for the fp32 fallback.
template <typename XT>
__device__ __forceinline__ float y_at(const XT* __restrict__ x, int64_t p, int dd, int d, int64_t ldx,
                                      const float* __restrict__ sc, const float* __restrict__ cs) {
    return dd < d ? fmaf(to_f32(x[p * ldx + dd]), sc[dd], -cs[dd]) : 0.0f;
}

template <int DP, int KB, typename XT, bool VEC, bool EM>
__global__ __launch_bounds__(64 * diag_split_waves(DP, KB), 1) void k_diag_split(
    const XT* __restrict__ x, int64_t n, int d, int64_t ldx, int k_real,
    const float* __restrict__ th_pi, const float* __restrict__ th_mu,
    const float* __restrict__ th_var, const double* __restrict__ chunk_part, int nch,
    const float* __restrict__ panel32, const float* __restrict__ shift,
    float* __restrict__ scale, double* __restrict__ part, double* __restrict__ part_ll,
    unsigned* __restrict__ done, double* __restrict__ ll_ws, double* __restrict__ ll_out,
    int* __restrict__ nonfinite_ll, float* __restrict__ out_lse, int* __restrict__ out_arg,
    int64_t tlo, int64_t thi, int seg_first, int topm, int* __restrict__ out_idx,
    float* __restrict__ out_gamma) {
    using S = SplitShape<DP, KB, XT>;
    constexpr int WAVES = S::kWaves, THREADS = S::kThreads;
    constexpr int KS = S::kKS, NCB = S::kNCB, EV = S::kEV, P = S::kPitch;
    constexpr int kRedFloats = WAVES * 16 * KB * 2 * DP;
    constexpr int kTileHalves = WAVES * 2 * S::kTile;
    constexpr int kSmemBytes = 2 * kTileHalves > 4 * kRedFloats ? 2 * kTileHalves : 4 * kRedFloats;
    __shared__ __attribute__((aligned(16))) uint4 smem[kSmemBytes / 16];
    __shared__ float cs_l[DP], sc_l[DP];
    __shared__ float s0red[WAVES][4][16 * KB];
    __shared__ double llred[THREADS];

    const int tid = threadIdx.x;
    const int lane = tid & 63, g = lane >> 4, j = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, kept scalar

    // this wave's run of the segment's tiles [tlo, thi) (wave-uniform; the
    // 64-bit division expands to vector code, so its results are moved back
    // to scalar registers)
    const int64_t tiles = thi - tlo;
    const int64_t nw = (int64_t)gridDim.x * WAVES, gw = (int64_t)blockIdx.x * WAVES + w;
    const int64_t tb = tiles / nw, tr = tiles % nw;
    const int64_t t0 = uniform64(tlo + gw * tb + (gw < tr ? gw : tr));
    const int nt = __builtin_amdgcn_readfirstlane((int)(tb + (gw < tr ? 1 : 0)));
    const int64_t tlast = t0 + nt - 1;

    const int col0 = (lane % S::kVPR) * EV;
    const bool colok = col0 < d;
    // offsets of this lane's vector slots from a tile's first row (bytes on
    // the vector path, elements of the row start otherwise); rows clamped
    // to the problem when it has fewer than 32 points
    uint32_t loff[S::kPer];
#pragma unroll
    for (int i = 0; i < S::kPer; ++i) {
        int r = row_of((lane + 64 * i) / S::kVPR);
        r = r < n ? r : (int)n - 1;
        loff[i] = VEC ? (uint32_t)(((int64_t)r * ldx + (colok ? col0 : 0)) * sizeof(XT))
                      : (uint32_t)((int64_t)r * ldx);
    }
    // First row of the 32 that tile t reads: the last, ragged tile is moved
    // back to end at row N (rows before its own start were counted by the
    // previous tile and are masked); problems under 32 points start at 0.
    auto tile_row = [&](int64_t t) {
        const int64_t p = t * kST;
        const int64_t pmax = n > kST ? n - kST : 0;
        return p < pmax ? p : pmax;
    };
    // the first tile's loads fly while the panel is built
    TileRegs<XT, DP, KB, VEC> ld;
    if (nt > 0) ld.load(x + tile_row(t0) * ldx, loff, d, lane);

    // ---- this step's split fp16 panel, built by every workgroup from the
    // prepared fp32 parameters (same inputs and code in all of them)
    constexpr int NC = 16 * KB;                     // padded components
    // threads per component: the largest power of two with NC * TPC <= THREADS
    constexpr int TPC = THREADS / NC >= 32 ? 32 : THREADS / NC >= 16 ? 16 : THREADS / NC >= 8 ? 8 : 4;
    constexpr int VPT = 2 * DP / TPC;               // panel values per thread
    float* const pab = reinterpret_cast<float*>(smem);   // [NC][2 DP]: a | b, y units / F_k
    float* const tmu = pab + NC * 2 * DP;                // [NC][DP] staged means
    float* const tvar = tmu + NC * DP;                   // [NC][DP] staged variances
    __shared__ float pf[NC], pc[NC], tpi[NC];
    // (0) the parameters into LDS in one round trip (padding: mu 0, var 1,
    // pi 0), and each component's log2 normaliser
    // c_k = log2(e) (log pi_k - 1/2 (D log 2pi + sum log var + sum (mu-c)^2/var))
    // from the per-chunk sums of the prepare / finalize kernel
    for (int e2 = tid; e2 < NC * DP; e2 += THREADS) {
        const int kb = e2 / DP, dd = e2 % DP;
        const bool ok = kb < k_real && dd < d;
        tmu[e2] = ok ? th_mu[(int64_t)kb * d + dd] : 0.0f;
        tvar[e2] = ok ? th_var[(int64_t)kb * d + dd] : 1.0f;
    }
    for (int kb = tid; kb < NC; kb += THREADS) {
        float cval = -INFINITY;   // padding component: weight 0
        float pk = 0.0f;
        if (kb < k_real) {
            pk = th_pi[kb];
            double sl = 0.0, sm = 0.0;
            for (int ch = 0; ch < nch; ++ch) {
                sl += chunk_part[((int64_t)kb * nch + ch) * 4 + 0];
                sm += chunk_part[((int64_t)kb * nch + ch) * 4 + 1];
            }
            cval = (float)((log((double)pk) - 0.5 * (d * kLog2Pi + sl + sm)) * kLog2e);
        }
        tpi[kb] = pk;
        pc[kb] = cval;
    }
    __syncthreads();
    // (1) per-dimension scale s (a power of two): the widest reach of the
    // components that hold weight, max_k |mu_k - c| + 4 sigma_k over
    // pi_k > 0, maps into [4, 8), so data within the model's spread has
    // |y| < 8 and the fp16 range (|y| < kSplitLim) leaves a factor of about
    // 28 for points beyond it; 1 when the reach is zero or not finite
    for (int dd = tid; dd < DP; dd += THREADS) {
        const float c = dd < d ? shift[dd] : 0.0f;
        float reach = 0.0f;
        for (int kb = 0; kb < k_real; ++kb) {
            const float v = tvar[kb * DP + dd];
            const float r = fabsf(tmu[kb * DP + dd] - c) + 4.0f * sqrtf(v > 0.0f ? v : 0.0f);
            if (tpi[kb] > 0.0f && isfinite(r)) reach = fmaxf(reach, r);
        }
        float sd = 1.0f;
        if (reach > 0.0f && isfinite(reach)) {
            int e = ilogbf(reach) - 2;
            e = e < -60 ? -60 : (e > 60 ? 60 : e);
            sd = ldexpf(1.0f, -e);
        }
        if (dd >= d) sd = 0.0f;
        sc_l[dd] = sd;
        cs_l[dd] = c * sd;
        if (blockIdx.x == 0) scale[dd] = dd < d ? sd : 1.0f;   // read by the reduction
    }
    __syncthreads();
    // (2) entries a = -1/2 log2(e) / (var s^2), b = log2(e) (mu - c) / (var s)
    // (fp32, a few roundings; s is a power of two, so dividing by it is
    // exact) and the component's power-of-two scale F_k (largest entry in
    // [2^14, 2^15))
    for (int kb = tid / TPC; kb < NC; kb += THREADS / TPC) {
        const int t = tid % TPC;
        float v[VPT];
        float mxa = 0.0f;
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int kk = t + TPC * i;
            const int dd = kk < DP ? kk : kk - DP;
            float val = 0.0f;
            if (kb < k_real && dd < d) {
                const float is = 1.0f / sc_l[dd];
                const float pr = (float)kLog2e / tvar[kb * DP + dd];
                val = kk < DP ? -0.5f * pr * is * is : (tmu[kb * DP + dd] - shift[dd]) * pr * is;
            }
            v[i] = val;
            if (isfinite(v[i])) mxa = fmaxf(mxa, fabsf(v[i]));
        }
#pragma unroll
        for (int o = TPC / 2; o > 0; o >>= 1) mxa = fmaxf(mxa, __shfl_xor(mxa, o));
        const int fe = mxa > 0.0f ? ilogbf(mxa) - 14 : 0;
        const float inv = ldexpf(1.0f, -fe);
#pragma unroll
        for (int i = 0; i < VPT; ++i) pab[kb * (2 * DP) + t + TPC * i] = v[i] * inv;
        if (t == 0) pf[kb] = ldexpf(1.0f, fe);
    }
    __syncthreads();
    // (3) this lane's B operands: component 16 b + j, K index 32 ks + 8 g + e
    half8 ph[KS][KB], pl[KS][KB];
    float cv[KB], fv[KB];
#pragma unroll
    for (int b = 0; b < KB; ++b) {
        const float* row = pab + (16 * b + j) * (2 * DP);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const float4 v0 = *reinterpret_cast<const float4*>(row + 32 * ks + 8 * g);
            const float4 v1 = *reinterpret_cast<const float4*>(row + 32 * ks + 8 * g + 4);
            uint32_t hw[4], lw[4];
            split2(v0.x, v0.y, hw[0], lw[0]);
            split2(v0.z, v0.w, hw[1], lw[1]);
            split2(v1.x, v1.y, hw[2], lw[2]);
            split2(v1.z, v1.w, hw[3], lw[3]);
            ph[ks][b] = __builtin_bit_cast(half8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
            pl[ks][b] = __builtin_bit_cast(half8, make_uint4(lw[0], lw[1], lw[2], lw[3]));
        }
        fv[b] = pf[16 * b + j];
        cv[b] = pc[16 * b + j];
    }
    float sv[EV], csv[EV];
#pragma unroll
    for (int e = 0; e < EV; ++e) {
        sv[e] = sc_l[col0 + e];
        csv[e] = cs_l[col0 + e];
    }
    __syncthreads();   // the panel area is reused by the tiles

    f32x4 acc[EM ? KB : 1][EM ? NCB : 1];
    float s0acc[KB];
#pragma unroll
    for (int b = 0; b < KB; ++b) {
        s0acc[b] = 0.0f;
        if constexpr (EM) {
#pragma unroll
            for (int c = 0; c < NCB; ++c) acc[b][c] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    double ll2 = 0.0;

    uint16_t* H = reinterpret_cast<uint16_t*>(smem) + w * 2 * S::kTile;
    uint16_t* L = H + S::kTile;

    // One tile: split-stage `ld`, issue the loads of tile q + 1 into it (they
    // land while this tile is computed), scores, softmax, statistics.
    auto step = [&](int q, TileRegs<XT, DP, KB, VEC>& ld) {
        const int64_t p0 = (t0 + q) * kST;   // first point this tile counts
        const int64_t pr = tile_row(t0 + q);  // first row it read
        const float mx = stage_tile<XT, DP, KB>(ld.raw, H, L, sv, csv, lane);
        const bool big = __ballot(mx > kSplitLim) != 0;   // wave-uniform
        {
            const int64_t tn = t0 + q + 1 <= tlast ? t0 + q + 1 : tlast;
            ld.load(x + tile_row(tn) * ldx, loff, d, lane);
        }
        wave_lds_fence();

        // ---- scores s[g2][b][r]: point 16 g2 + 4 g + r, component 16 b + j (base 2)
        float s[2][KB][4];
        if (!big) {
            f32x4 sa[2][KB];
#pragma unroll
            for (int g2 = 0; g2 < 2; ++g2)
#pragma unroll
                for (int b = 0; b < KB; ++b) sa[g2][b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int g2 = 0; g2 < 2; ++g2) {
                    const int o = uoff<P>(16 * g2 + j, 4 * ks + g);
                    const half8 ah = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(H + o));
                    const half8 al = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(L + o));
#pragma unroll
                    for (int b = 0; b < KB; ++b) {
                        sa[g2][b] = mfma_f16(ah, ph[ks][b], sa[g2][b]);
                        sa[g2][b] = mfma_f16(ah, pl[ks][b], sa[g2][b]);
                        sa[g2][b] = mfma_f16(al, ph[ks][b], sa[g2][b]);
                    }
                }
            }
#pragma unroll
            for (int g2 = 0; g2 < 2; ++g2)
#pragma unroll
                for (int b = 0; b < KB; ++b)
#pragma unroll
                    for (int r = 0; r < 4; ++r) s[g2][b][r] = fmaf(sa[g2][b][r], fv[b], cv[b]);
        } else {
            // fp32 fallback: [x'^2 | x'] . [a ; b] on v_mfma_f32_16x16x4f32 with
            // x' = x - c read back from global memory and the fp32 panel
#pragma unroll
            for (int g2 = 0; g2 < 2; ++g2) {
                int64_t p = pr + 16 * g2 + j;
                p = p < n ? p : n - 1;
                f32x4 sb[KB];
#pragma unroll
                for (int b = 0; b < KB; ++b) sb[b] = f32x4{cv[b], cv[b], cv[b], cv[b]};
#pragma unroll 1
                for (int st = 0; st < DP / 4; ++st) {
                    const int dd = g * (DP / 4) + st;
                    const float xs = dd < d ? to_f32(x[p * ldx + dd]) - shift[dd] : 0.0f;
#pragma unroll
                    for (int b = 0; b < KB; ++b) {
                        sb[b] = mfma16x16x4(xs * xs, panel32[((st * 2) * KB + b) * 64 + lane], sb[b]);
                        sb[b] = mfma16x16x4(xs, panel32[((st * 2 + 1) * KB + b) * 64 + lane], sb[b]);
                    }
                }
#pragma unroll
                for (int b = 0; b < KB; ++b)
#pragma unroll
                    for (int r = 0; r < 4; ++r) s[g2][b][r] = sb[b][r];
            }
        }

        // ---- base-2 log-sum-exp and responsibilities (fp32)
        // rows [lo, hi) of the 32 read are this tile's points
        const int lo = (int)(p0 - pr);
        const int hi = n - pr < kST ? (int)(n - pr) : kST;
        float m[2][4], z[2][4];
        bool valid[2][4];
        float tll = 0.0f;
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float mv = s[g2][0][r];
#pragma unroll
                for (int b = 1; b < KB; ++b) mv = fmaxf(mv, s[g2][b][r]);
                m[g2][r] = row16_max(mv);
            }
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float zz = 0.0f;
#pragma unroll
                for (int b = 0; b < KB; ++b) {
                    const float e = fast_exp2(s[g2][b][r] - m[g2][r]);
                    if constexpr (EM) s[g2][b][r] = e;   // s now holds the exponentials
                    zz += e;
                }
                z[g2][r] = row16_sum(zz);
                const int row = 16 * g2 + 4 * g + r;
                valid[g2][r] = row >= lo && row < hi;
                const float lse2 = m[g2][r] + fast_log2(z[g2][r]);
                tll += valid[g2][r] ? lse2 : 0.0f;
                if constexpr (!EM) {
                    const int64_t pt = pr + 16 * g2 + 4 * g + r;
                    if (out_lse != nullptr && j == 0 && valid[g2][r])
                        out_lse[pt] = (float)((double)lse2 * kLn2);
                    if (out_arg != nullptr) {
                        int best = 0x7fffffff;
#pragma unroll
                        for (int b = KB - 1; b >= 0; --b)
                            if (s[g2][b][r] == m[g2][r] && 16 * b + j < k_real) best = 16 * b + j;
                        best = row16_min_i(best);
                        if (j == 0 && valid[g2][r]) out_arg[pt] = best;
                    }
                    if (topm > 0) {
                        // the topm largest scores of the point (lower component first
                        // on ties): repeated max over the 16 lanes of the row, the
                        // lane holding the winner drops it from its candidates
                        float cur[KB];
#pragma unroll
                        for (int b = 0; b < KB; ++b) cur[b] = 16 * b + j < k_real ? s[g2][b][r] : -INFINITY;
                        for (int i = 0; i < topm; ++i) {
                            float bv = -INFINITY;
                            int bk = 0x7fffffff;
#pragma unroll
                            for (int b = 0; b < KB; ++b)
                                if (cur[b] > bv) {
                                    bv = cur[b];
                                    bk = 16 * b + j;
                                }
                            const float mv = row16_max(bv);
                            const int kb = row16_min_i(bv == mv ? bk : 0x7fffffff);
#pragma unroll
                            for (int b = 0; b < KB; ++b)
                                if (16 * b + j == kb) cur[b] = -INFINITY;
                            if (j == 0 && valid[g2][r]) {
                                const bool live = mv != -INFINITY;
                                out_idx[pt * topm + i] = live ? kb : -1;
                                out_gamma[pt * topm + i] = live ? fast_exp2(mv - lse2) : 0.0f;
                            }
                        }
                    }
                }
            }
        ll2 += (double)tll;

        if constexpr (EM) {
            // gamma (fp32) in s; s0 in fp32
#pragma unroll
            for (int g2 = 0; g2 < 2; ++g2)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float inv = valid[g2][r] ? __builtin_amdgcn_rcpf(z[g2][r]) : 0.0f;
#pragma unroll
                    for (int b = 0; b < KB; ++b) s[g2][b][r] *= inv;
                }
#pragma unroll
            for (int b = 0; b < KB; ++b)
                s0acc[b] += ((s[0][b][0] + s[0][b][1]) + (s[0][b][2] + s[0][b][3])) +
                            ((s[1][b][0] + s[1][b][1]) + (s[1][b][2] + s[1][b][3]));

            if (!big) {
                // A operand of gamma^T (components x 32 points): K index 8g + e is
                // point 4g + e of group 0 (e < 4) or 4g + e - 4 of group 1
                half8 gh[KB], gl[KB];
#pragma unroll
                for (int b = 0; b < KB; ++b) {
                    uint32_t hw[4], lw[4];
#pragma unroll
                    for (int q2 = 0; q2 < 4; ++q2) {
                        const int g2 = q2 >> 1, r = 2 * (q2 & 1);
                        split2(s[g2][b][r], s[g2][b][r + 1], hw[q2], lw[q2]);
                    }
                    gh[b] = __builtin_bit_cast(half8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
                    gl[b] = __builtin_bit_cast(half8, make_uint4(lw[0], lw[1], lw[2], lw[3]));
                }
                // B operand (32 points x 16 columns) by transposed reads: lane
                // (g, i) addresses row 4g + i / 4 (and 16 + ...), column 16 cb + 4 (i % 4)
                const int rr = 4 * g + (j >> 2), cq = 4 * (j & 3);
                half8 bh[NCB], bl[NCB];
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    const int c0 = 16 * cb + cq;
                    const int oa = uoff<P>(rr, c0 >> 3) + (c0 & 7);
                    const int ob = uoff<P>(rr + 16, c0 >> 3) + (c0 & 7);
                    const uint2 ha = tr16(H + oa), hb = tr16(H + ob);
                    const uint2 la = tr16(L + oa), lb = tr16(L + ob);
                    bh[cb] = __builtin_bit_cast(half8, make_uint4(ha.x, ha.y, hb.x, hb.y));
                    bl[cb] = __builtin_bit_cast(half8, make_uint4(la.x, la.y, lb.x, lb.y));
                }
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                    for (int b = 0; b < KB; ++b) {
                        acc[b][cb] = mfma_f16(gh[b], bh[cb], acc[b][cb]);
                        acc[b][cb] = mfma_f16(gh[b], bl[cb], acc[b][cb]);
                        acc[b][cb] = mfma_f16(gl[b], bh[cb], acc[b][cb]);
                    }
                // reads run two column blocks ahead of the MFMAs, so the LDS
                // latency is paid about once per tile, not once per block
                __builtin_amdgcn_sched_group_barrier(0x100, NCB > 1 ? 8 : 4, 0);
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 3 * KB, 0);
                    if (cb + 2 < NCB) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
                }
            } else {
                // fp32 fallback: [S2 | S1] += gamma^T [y^2 | y], y read back from
                // global memory, v_mfma_f32_16x16x4f32 (same accumulator layout)
#pragma unroll
                for (int db = 0; db < DP / 16; ++db) {
                    const int dd = 16 * db + j;
#pragma unroll
                    for (int g2 = 0; g2 < 2; ++g2)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            int64_t p = pr + 16 * g2 + 4 * g + r;
                            p = p < n ? p : n - 1;
                            const float y = y_at(x, p, dd, d, ldx, sc_l, cs_l);
#pragma unroll
                            for (int b = 0; b < KB; ++b) {
                                acc[b][db] = mfma16x16x4(s[g2][b][r], y * y, acc[b][db]);
                                acc[b][DP / 16 + db] = mfma16x16x4(s[g2][b][r], y, acc[b][DP / 16 + db]);
                            }
                        }
                }
            }
        }
        wave_lds_fence();   // this tile's LDS reads before the next staging writes
    };

    for (int q = 0; q < nt; ++q) step(q, ld);

    // ---- one fp64 partial per workgroup, waves summed in a fixed order
    // LL: fixed-order tree over the workgroup (the lanes j == 0 hold the sums)
    const double ll_wg = block_sum_f64((j == 0) ? ll2 : 0.0, llred);   // synchronises
    float* red = reinterpret_cast<float*>(smem);
    if constexpr (EM) {
        // acc[b][cb] lane (g, j): components 16 b + 4 g + r, column 16 cb + j of [y^2 | y]
#pragma unroll
        for (int b = 0; b < KB; ++b)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int comp = 16 * b + 4 * g + r;
                    red[(w * 16 * KB + comp) * (2 * DP) + 16 * cb + j] = acc[b][cb][r];
                }
#pragma unroll
        for (int b = 0; b < KB; ++b) s0red[w][g][16 * b + j] = s0acc[b];
    }
    __syncthreads();
    const int64_t wg = blockIdx.x;
    if constexpr (EM) {
        // partial columns: [s0, S1_0, S2_0, S1_1, S2_1, ...] (moments of y about c).
        // s0 per component first (its 4 WAVES terms summed once, not in the
        // column loop, where its lanes would hold up the rest of their wave)
        __shared__ double s0sum[16 * KB];
        for (int k = tid; k < k_real; k += THREADS) {
            double v = 0.0;
            for (int w2 = 0; w2 < WAVES; ++w2)
                for (int g2 = 0; g2 < 4; ++g2) v += (double)s0red[w2][g2][k];
            s0sum[k] = v;
        }
        __syncthreads();
        const int ncol = 1 + 2 * d;
        for (int e2 = tid; e2 < k_real * ncol; e2 += THREADS) {
            const int k = e2 / ncol, c = e2 % ncol;
            double v;
            if (c == 0) {
                v = s0sum[k];
            } else {
                const int dd = (c - 1) >> 1, mom = (c - 1) & 1;
                const int col = mom == 0 ? DP + dd : dd;   // S1 <- y, S2 <- y^2
                double v0 = 0.0, v1 = 0.0;   // even and odd waves, all reads issued together
#pragma unroll
                for (int w2 = 0; w2 < WAVES; w2 += 2) {
                    v0 += (double)red[(w2 * 16 * KB + k) * (2 * DP) + col];
                    v1 += (double)red[((w2 + 1) * 16 * KB + k) * (2 * DP) + col];
                }
                v = v0 + v1;
            }
            double* o = part + (wg * k_real + k) * ncol + c;
            // later segments add to the slot; streamed past the L2
            __builtin_nontemporal_store(seg_first ? v : *o + v, o);
        }
    }
    // LL of the whole pass: the last workgroup to finish sums the
    // per-workgroup values in a fixed order.  Each value is stored as a
    // device-scope atomic (written through to the level every XCD sees) and
    // waited for before the count moves, and the last workgroup reads them
    // with device-scope atomic loads: no L2 write-back or invalidation is
    // needed for them (the partial slots above are read by the next kernel,
    // after this one has ended).  The count returns to zero for the next
    // launch.
    __shared__ int last_wg;
    if (tid == 0) {
        const double llv = seg_first ? ll_wg * kLn2 : part_ll[wg] + ll_wg * kLn2;
        __hip_atomic_store(&part_ll[wg], llv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);   // the store is done before the count moves
        asm volatile("" ::: "memory");
        const unsigned prev = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last_wg = prev == gridDim.x - 1;
    }
    __syncthreads();
    if (last_wg) {
        double v = 0.0;
        for (int p = tid; p < (int)gridDim.x; p += THREADS)
            v += __hip_atomic_load(&part_ll[p], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        v = block_sum_f64(v, llred);
        if (tid == 0) {
            *ll_ws = v;
            if (ll_out != nullptr) *ll_out = v;
            *nonfinite_ll = isfinite(v) ? 0 : 1;
            *done = 0u;
        }
    }
}

// EM: the pass in segments of at most seg_tiles tiles per wave (each closes
// the waves' fp32 runs into the fp64 partial slots); E-step alone: one pass.
template <int DP, int KB, typename XT, bool VEC, bool EM>
hipError_t launch_t(const Plan& p, const DiagWs& w, const void* x, int grid, double* ll_out,
                    float* lse, int* arg, const DiagTopm& tm, hipStream_t s) {
    constexpr int W = diag_split_waves(DP, KB);
    const int64_t tiles = (p.n + kST - 1) / kST;
    const int64_t M = p.seg_tiles > 0 ? p.seg_tiles : kDiagSegTiles;
    const int64_t per = (int64_t)grid * W * M;
    const int64_t nseg = EM ? (tiles + per - 1) / per : 1;
    const int64_t len = nseg > 1 ? (tiles + nseg - 1) / nseg : tiles;
    for (int64_t i = 0; i < (nseg < 1 ? 1 : nseg); ++i) {
        const int64_t lo = i * len, hi = lo + len < tiles ? lo + len : tiles;
        hipLaunchKernelGGL((k_diag_split<DP, KB, XT, VEC, EM>), dim3(grid), dim3(64 * W), 0, s,
                           (const XT*)x, p.n, (int)p.d, p.ldx, (int)p.k, w.pi, w.mu, w.var,
                           w.chunk_part, diag_chunks(p), w.panel, w.shift, w.scale, w.part, w.part_ll,
                           (unsigned*)w.done, w.ll, ll_out, w.nonfinite_ll, lse, arg, lo, hi,
                           i == 0 ? 1 : 0, tm.m, tm.idx, tm.gamma);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int DP, int KB, bool EM>
hipError_t launch_x(const Plan& p, const DiagWs& w, const void* x, bool vec, int grid,
                    double* ll_out, float* lse, int* arg, const DiagTopm& tm, hipStream_t s) {
    switch (p.xdt) {
        case GMM_F32:
            return vec ? launch_t<DP, KB, float, true, EM>(p, w, x, grid, ll_out, lse, arg, tm, s)
                       : launch_t<DP, KB, float, false, EM>(p, w, x, grid, ll_out, lse, arg, tm, s);
        case GMM_BF16:
            return vec ? launch_t<DP, KB, bf16_t, true, EM>(p, w, x, grid, ll_out, lse, arg, tm, s)
                       : launch_t<DP, KB, bf16_t, false, EM>(p, w, x, grid, ll_out, lse, arg, tm, s);
        default:
            return vec ? launch_t<DP, KB, _Float16, true, EM>(p, w, x, grid, ll_out, lse, arg, tm, s)
                       : launch_t<DP, KB, _Float16, false, EM>(p, w, x, grid, ll_out, lse, arg, tm, s);
    }
}

bool x_vec_ok(const Plan& p, const void* x) {
    const int es = p.xdt == GMM_F32 ? 4 : 2;
    const int ev = 16 / es;
    return ((uintptr_t)x % 16 == 0) && ((p.ldx * es) % 16 == 0) && (p.d % ev == 0);
}

}  // namespace

hipError_t diag_launch_split(const Plan& p, const DiagWs& w, const void* x, bool em, int grid,
                             double* ll_out, float* lse, int* arg, const DiagTopm& tm,
                             hipStream_t s) {
    const bool vec = x_vec_ok(p, x);
#define CASE(DP_, KB_)                                                                          \
    if (p.dp == DP_ && p.kb == KB_)                                                             \
        return em ? launch_x<DP_, KB_, true>(p, w, x, vec, grid, ll_out, lse, arg, tm, s)      \
                  : launch_x<DP_, KB_, false>(p, w, x, vec, grid, ll_out, lse, arg, tm, s);
    GMM_DIAG_SHAPES(CASE)
#undef CASE
    return hipErrorInvalidValue;
}

}  // namespace gmm
