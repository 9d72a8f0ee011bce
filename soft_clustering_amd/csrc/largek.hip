// Large-K Gaussian mixtures (isotropic or diagonal covariance, X stored in
// bf16 or fp16): fused E-step + M-step statistics on fp16 MFMA
// (v_mfma_f32_32x32x16_f16, fp32 accumulation), fp32 softmax.
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
//   diag: S_k = F (y'^2 . A_k + y' . B_k + C_k)
//   iso:  S_k = F (y' . W_k + P_k |y|^2 2^-g + C_k)
// with one power-of-two panel scale F for all components.  The contraction
// runs over [y'^2 | y' | 16 bias slots] (diag) or [y' | 16 bias slots] (iso):
// the bias slots hold C_k (and P_k) split into fp16 high and low parts
// against constant ones (and |y|^2 2^-g split the same way, fp32 accurate), so
// the MFMA returns the whole score and the vector unit only forms exp2.
//
// Layout: the score MFMA has the components as rows and the 32 points of a
// tile as columns, so each lane holds one point's scores for 16 components
// per block and the per-point max / sum is mostly lane-local (one exchange
// between the two wave halves).  Responsibilities go through a wave-private
// LDS tile [point][component] and come back, with ds_read_b64_tr_b16, as the
// components-by-points A operand of the statistics MFMA; the B operand
// (points by features) is read the same way from the row-major tile of X.
// s0 (and the isotropic sum gamma |y|^2) come from one v_mfma_f32_16x16x32_f16
// per 16 components against a [1, |y|^2] column pair.
//
// Work split: a workgroup owns a slice of 256 components, 64 per wave; each
// wave keeps its components' panel in registers.  32-point tiles are staged
// once per workgroup into LDS (y', y'^2 and the bias slots, row-major),
// double buffered: one barrier per tile plus one for the exchange of the
// waves' per-point (max, sum) in the modes that normalise.  The slices of one
// point chunk are mapped to one XCD so X is read from HBM once and re-read
// from that L2.

#include <type_traits>

#include "largek_internal.h"

namespace gmm {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

constexpr int kT = kLkT;
constexpr float kLn2f = 0.69314718055994530942f;

// LDS layouts, chosen by measuring bank conflicts on gfx950 (SQ_LDS_BANK_CONFLICT
// over each access pattern): tile of X: rows at a pitch of an odd multiple of
// 16 bytes (mod 256), which keeps the 16-byte score-operand reads of 32 rows
// and the staging writes conflict-free; responsibility tile: 64 components
// (128 bytes) per point with the 8-byte units XOR-swizzled by
// ((r & 3) << 2 | (r >> 2) & 3), conflict-free for the 32-row unit writes and
// the transposed reads.
constexpr int row_pad(int inner) { return (24 - inner % 128 + 128) % 128; }

template <int KW>
__device__ __forceinline__ int g_swz(int r) {
    if constexpr (KW == 64) return ((r & 3) << 2) | ((r >> 2) & 3);
    // 32 components (64-byte rows, 8 units): bits 2..4 of r, bit 3 in the top
    return (((r >> 3) & 1) << 2) | (((r >> 2) & 1) << 1) | ((r >> 4) & 1);
}

template <int COV, int DP>
struct LkShape {
    static constexpr bool kIso = COV == GMM_COV_ISO;
    static constexpr int kFeat = kIso ? DP : 2 * DP;     // statistics features
    static constexpr int kInner = kFeat + 16;            // + bias slots
    static constexpr int kKS = kInner / 16;              // 32x32x16 steps per score
    static constexpr int kRowY = kInner + row_pad(kInner);
    static constexpr int kNFB = kFeat / 32;              // 32-feature blocks
    static constexpr int kCB = DP / 8;                   // 8-column blocks per row of X
    static constexpr int kItems = kT * kCB;
    static constexpr int kFCh = kFeat / 8;               // 16-byte feature chunks per row
    // halves offset of 16-byte chunk c of row r
    static __device__ __forceinline__ int ych(int r, int c) { return r * kRowY + 8 * c; }
};

// halves offset of 4-half unit u of row r in the responsibility tile (KW components per row)
template <int KW>
__device__ __forceinline__ int gch(int r, int u) { return r * KW + 4 * (u ^ g_swz<KW>(r)); }

__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
    const half2v h = {(_Float16)lo, (_Float16)hi};       // v_cvt_pk_f16_f32, round to nearest even
    return __builtin_bit_cast(uint32_t, h);
}

// MFMAs with their accumulators in VGPRs, for the statistics kernels that run
// one wave per SIMD.  There the compiler gives every MFMA an AGPR accumulator,
// and the scores (32 registers) and s0 (16) then share the 256 AGPRs with the
// 256 statistics accumulators: it copies scores out for the softmax and swaps
// statistics in and out around their MFMAs, 128 register moves per tile.  In
// inline asm the accumulator is a VGPR operand.  The compiler does not see the
// MFMA inside the asm, so the wait states it would insert are written out: a
// few before each (a VALU write of an operand just before an MFMA needs them)
// and `mfma_v_settle` (24) after the last one, before any other instruction
// touches the results (a 32x32x16 result needs 11 before a VALU reads it).
// The "+v" operands of the settle make every later use depend on it.
// (first: the accumulator starts at zero; a constant once the loop unrolls)
__device__ __forceinline__ void mfma32_v(f32x16& d, const half8& a, const half8& b, bool first) {
    if (first)
        asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
    else
        asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma16_v(f32x4& d, const half8& a, const half8& b) {
    asm volatile("s_nop 4\n\tv_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v_settle(f32x16& x, f32x16& y) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(x), "+v"(y));
}
__device__ __forceinline__ void mfma_v_settle(f32x4& x, f32x4& y, f32x4& z, f32x4& u) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(x), "+v"(y), "+v"(z), "+v"(u));
}

template <bool BF16>
__device__ __forceinline__ float h16_to_f32(uint32_t bits16) {
    if constexpr (BF16) return __uint_as_float(bits16 << 16);
    const uint16_t b = (uint16_t)bits16;
    return (float)__builtin_bit_cast(_Float16, b);
}

// Eight consecutive 16-bit elements of one row (zeros beyond column d on the
// element-wise path; the vector path needs d % 8 == 0 and col < d).  The
// path is a template argument: a run-time branch joins the two paths'
// registers, and the join waits for the prefetch loads to land.
template <bool VEC>
__device__ __forceinline__ uint4 load8(const uint16_t* __restrict__ row, int col, int d) {
    if constexpr (VEC) return *reinterpret_cast<const uint4*>(row + col);
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t lo = col + 2 * q < d ? row[col + 2 * q] : 0u;
        const uint32_t hi = col + 2 * q + 1 < d ? row[col + 2 * q + 1] : 0u;
        w[q] = lo | (hi << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// ds_read_b64_tr_b16: in each group of 16 lanes, lane i' reads 4 halves of
// row (i' / 4) at column 4 (i' % 4) (addresses as given); lane i receives
// column i of the 4 rows.  Two such reads give the 8 consecutive K values of
// an MFMA operand for rows of K stored contiguously along the M/N index.
__device__ __forceinline__ uint2 tr16(const uint16_t* p) {
    const short4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)((lds_u16*)p));
    return __builtin_bit_cast(uint2, v);
}

template <int COV, int DP, int MODE_ARG, bool BF16, bool VEC>
__global__ __launch_bounds__(lk_threads(MODE_ARG, COV), lk_wg_per_cu(MODE_ARG)) void k_lk(const LkArgs a) {
    constexpr int MODE = MODE_ARG & (kLkArg - 1);
    constexpr bool want_arg = (MODE_ARG & kLkArg) != 0 && (MODE == LK_SWEEP1 || MODE == LK_FUSED_E);
    constexpr int SPW = lk_slices_per_wg(MODE_ARG);   // slices per workgroup (2: sweep 1 only)
    static_assert(SPW == 1 || MODE == LK_SWEEP1, "paired slices: sweep 1 only");
    constexpr int WV = lk_waves(MODE, COV);     // waves per slice
    constexpr int WT = WV * SPW;                // waves per workgroup
    constexpr int KW = kLkSlice / WV;           // components per wave
    constexpr int CB = KW / 32;                 // 32-component blocks per wave
    constexpr int NT = 64 * WT;                 // threads per workgroup
    using Sh = LkShape<COV, DP>;
    constexpr bool kIso = Sh::kIso;
    constexpr int KS = Sh::kKS, NFB = Sh::kNFB, RY = Sh::kRowY;
    static_assert(KW == 64 || KW == 32, "responsibility tile layout: 32 or 64 components per wave");
    constexpr int RG = KW;                      // halves per row of the responsibility tile
    constexpr int IPT = (Sh::kItems + NT - 1) / NT;   // staging items per thread
    constexpr bool kStats = MODE == LK_FUSED_EM || MODE == LK_SWEEP2;
    constexpr bool kExchange = MODE != LK_SWEEP2 && MODE != LK_TOPM;
    constexpr bool kTopm = MODE == LK_TOPM;
    // diagonal statistics at D = 128: the accumulators fill the AGPRs, so the
    // y'^2 half of the panel (KL steps) is kept in LDS instead of registers
    constexpr bool kTight = kStats && !kIso && DP == 128;
    constexpr int KL = kTight ? DP / 16 : 0;   // panel steps [0, KL) and the bias step in LDS
    constexpr int KR = KS - 1 - KL;            // panel steps in registers: [KL, KS - 1)
    // one wave per SIMD there: scores and s0 accumulate in VGPRs (mfma32_v)
    constexpr bool kAsmAcc = kTight;

    // tiles of X in LDS: double buffered; the fused E+M mode keeps three, so
    // that the tile being staged is never one a slower wave still reads for
    // its statistics and the exchange barrier is the only one per tile
    constexpr int NYB = (kExchange && kStats) ? 3 : 2;
    __shared__ __attribute__((aligned(16))) uint16_t ybuf[NYB][kT * RY];
    __shared__ __attribute__((aligned(16))) uint16_t gbuf[kStats ? WV : 1][kStats ? kT * RG : 8];
    __shared__ __attribute__((aligned(16))) uint16_t yh_t[NYB][kT];   // iso: |y|^2 2^-g, fp16
    __shared__ uint4 plds[WT][CB][KL + 1][64];   // LDS-resident steps of each wave's panel
    __shared__ float2 dsc_l[DP];       // [e][8-column block], column 8 block + e: iso (c, s), diag (s, -c s)
    // the modes that exchange per-point values between waves: one barrier per
    // tile (the exchange's); the exchange buffers alternate between tiles so
    // that a wave writing the next tile's values cannot overwrite values
    // another wave still reads
    constexpr bool kOneBarrier = kExchange;
    constexpr int NXB = kOneBarrier ? 2 : 1;
    __shared__ float2 wpart_b[NXB][WT][kT];   // per-wave (max, sum) of each point, base-2 score units
    __shared__ int warg_b[NXB][WT][kT];
    __shared__ double llred[NT];
    // top-m mode: the slice's base-2 scores of the tile, each point's partial
    // lists (8 threads per point, 32 components each) and the running list
    // of the earlier slices (list 8), and the heads of the 9 sorted lists
    __shared__ float stile[kTopm ? kT : 1][kTopm ? kLkSlice + 1 : 1];
    __shared__ float2 cand[kTopm ? kT : 1][kTopm ? 9 : 1][kTopm ? kLkMaxTopm : 1];
    __shared__ int8_t chead[kTopm ? kT : 1][kTopm ? 9 : 1];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wl = w % WV, w0 = w - wl;                 // wave within its slice, the slice's first wave
    const int pn = lane & 31, hf = lane >> 5;           // point column, wave half
    const int gq = lane >> 4, gi = lane & 15;           // 16-lane group, lane in group
    const int G = gridDim.x, S = a.S;
    int slice, chunk;
    if constexpr (kTopm) {
        slice = a.topm_slice;
        chunk = blockIdx.x;
    } else {
        // workgroup b -> (slice group, chunk); the groups of one chunk share an XCD
        const int b = blockIdx.x, Sg = S / SPW;
        int sg;
        if (G % (8 * Sg) == 0) {
            const int r = b >> 3;
            sg = r % Sg;
            chunk = (r / Sg) * 8 + (b & 7);
        } else {
            sg = b % Sg;
            chunk = b / Sg;
        }
        slice = sg * SPW + w / WV;
    }
    const int nchunks = kTopm ? G : G / (S / SPW);
    const int kbase = slice * kLkSlice + wl * KW;
    const int64_t n = a.n;
    const int d = a.d;
    const float F = a.prm[0];                   // panel scale 2^f
    const float ysc = a.prm[1];                 // |y|^2 scale 2^-g (isotropic)
    // components scored exactly outside the panel (their per-point LSE, best
    // score and its component are already in xlse / xmax / xarg)
    constexpr bool kXc = MODE == LK_FUSED_EM || MODE == LK_FUSED_E || MODE == LK_TOPM;
    const int nxc = (kXc && a.xc_n != nullptr) ? *a.xc_n : 0;

    // ---- this wave's panel: A operand, row = component, K = inner; steps
    // [KL, KS - 1) in registers, the others (the bias step, and at KL > 0 the
    // y'^2 half) in LDS, read once per tile
    half8 pnl[CB][KR > 0 ? KR : 1];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const uint4 v = a.panel[((int64_t)ks * a.nblk + kbase / 32 + cb) * 64 + lane];
            if (ks >= KL && ks < KS - 1) pnl[cb][ks - KL] = __builtin_bit_cast(half8, v);
            else plds[w][cb][ks < KL ? ks : KL][lane] = v;
        }
    }
    for (int i = tid; i < DP; i += NT) {
        const float2 cs = a.dsc[i];   // (c, s)
        dsc_l[(i % 8) * Sh::kCB + i / 8] = kIso ? cs : make_float2(cs.y, -cs.x * cs.y);
    }

    // ---- this chunk's tiles of the segment [tlo, thi)
    const int64_t tiles = a.thi - a.tlo;
    const int64_t tb = tiles / nchunks, tr = tiles % nchunks;
    const int64_t t0 = a.tlo + chunk * tb + (chunk < tr ? chunk : tr);
    const int64_t t1 = t0 + tb + (chunk < tr ? 1 : 0);

    f32x16 acc[kStats ? CB : 1][kStats ? NFB : 1];
    f32x4 aux[kStats ? KW / 16 : 1];
    if constexpr (kStats) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[cb][fb][r] = 0.0f;
#pragma unroll
        for (int b = 0; b < KW / 16; ++b) aux[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    double ll2 = 0.0;
    float rng = 0.0f;   // iso: largest |y|^2 2^-g staged (clamped above the fp16 maximum)
    half2v rq = {(_Float16)0.0f, (_Float16)0.0f};   // diag: largest fp16 (y')^2 staged (inf: out of range)

    // ---- staging: item (row, 8-column block); the kCB items of a row sit in
    // consecutive lanes and every item of a thread has the same column block.
    // Rows beyond N repeat the tile's last row (their responsibilities are
    // zeroed and their LSE is not written); columns beyond D read as zero.
    // The conversion is straight-line code, so it can be interleaved with the
    // score MFMAs of the previous tile.
    static_assert(NT % Sh::kCB == 0, "column block fixed per thread");
    const uint16_t* xb = reinterpret_cast<const uint16_t*>(a.x);
    const int cbk = tid % Sh::kCB, col0 = 8 * cbk;
    const bool col_ok = col0 < d;
    uint4 raw[IPT];
#pragma unroll
    for (int q = 0; q < IPT; ++q) raw[q] = make_uint4(0, 0, 0, 0);
    float lse_nx = 0.0f;

    auto load_tile = [&](int64_t t) {
        const int64_t p0 = t * kT;
        const int64_t left = n - p0;
        const int last = (left >= kT ? kT : (int)left) - 1;
#pragma unroll
        for (int q = 0; q < IPT; ++q) {
            const int it = tid + NT * q;
            if (Sh::kItems % NT == 0 || it < Sh::kItems) {
                const int r = it / Sh::kCB;
                raw[q] = load8<VEC>(xb + (p0 + (r < last ? r : last)) * a.ldx, col_ok ? col0 : 0, d);
            }
        }
    };
    // sweep 2: merged LSE of point pn of tile t (+inf beyond N: gamma = 0)
    auto load_lse = [&](int64_t t) {   // clamped index and a select: no branch around the load
        const int64_t p = t * kT + pn;
        const float v = a.lse_in[p < n ? p : n - 1];
        return p < n ? v : INFINITY;
    };

    // Top-m of the tile's points over this slice, merged with the running
    // list of the slices before it (the outputs).  An entry is better when its
    // score is larger, or equal with a lower component index; components
    // scoring -inf (zero weight, padding) are never listed.  Thread (p, q),
    // p = tid / 8, first selects the best m of components 32 q .. 32 q + 31;
    // thread p < 32 then merges the 8 sorted lists and the running one.
    auto topm_tile = [&](int64_t prow) {
        const int m = a.topm;
        {
            const int pt = tid >> 3, q = tid & 7;
            uint32_t taken = 0;
            for (int i = 0; i < m; ++i) {
                float bv = -INFINITY;
                int bc = -1;
                for (int c = 0; c < 32; ++c) {
                    const float v = stile[pt][32 * q + c];
                    if (!((taken >> c) & 1u) && v > bv) {
                        bv = v;
                        bc = c;
                    }
                }
                if (bc >= 0) taken |= 1u << bc;
                const int kg = bc >= 0 ? slice * kLkSlice + 32 * q + bc : -1;
                cand[pt][q][i] = make_float2(bv, __int_as_float(kg));
            }
            if (q == 0) {
                const int64_t pg = prow + pt;
                for (int i = 0; i < m; ++i) {
                    float2 e = make_float2(-INFINITY, __int_as_float(-1));
                    if ((slice > 0 || nxc > 0) && pg < n) {
                        const int kr = a.out_idx[pg * m + i];
                        if (kr >= 0) e = make_float2(a.out_gamma[pg * m + i], __int_as_float(kr));
                    }
                    cand[pt][8][i] = e;
                }
            }
            if (tid < kT)
                for (int l = 0; l < 9; ++l) chead[tid][l] = 0;
        }
        __syncthreads();
        if (tid < kT) {
            const int pt = tid;
            const int64_t pg = prow + pt;
            const bool last = slice == a.S - 1;
            const float lse2 = (last && pg < n) ? a.lse_in[pg] : 0.0f;
            for (int i = 0; i < m; ++i) {
                float bv = -INFINITY;
                int bk = -1, bl = -1;
                for (int l = 0; l < 9; ++l) {
                    const int h = chead[pt][l];
                    if (h >= m) continue;
                    const float2 e = cand[pt][l][h];
                    const int k = __float_as_int(e.y);
                    if (k >= 0 && (e.x > bv || (e.x == bv && (bk < 0 || k < bk)))) {
                        bv = e.x;
                        bk = k;
                        bl = l;
                    }
                }
                if (bl >= 0) chead[pt][bl] = (int8_t)(chead[pt][bl] + 1);
                if (pg < n) {
                    a.out_idx[pg * m + i] = bk;
                    a.out_gamma[pg * m + i] = bk < 0 ? 0.0f : (last ? fast_exp2(bv - lse2) : bv);
                }
            }
        }
    };

    // isotropic bias slots of a row, [yh, yl, yh, 1, 1, 0...]: this lane's 16 / kCB of them
    constexpr int kSlots = 16 / Sh::kCB;
    constexpr int kPairs = 4 * IPT;       // staging steps: two columns of one item each
    uint32_t hy[4], hq[4];                // packed y' and y'^2 of the current item
    float ss = 0.0f;                      // isotropic: partial |y|^2 of the current item
    // this thread's 8 (centre, scale) pairs: read once per kernel and kept in
    // registers where the registers allow (otherwise once per tile).  Read
    // per tile, the compiler places the reads where the staging uses them,
    // after the operand reads issued ahead, and each wait for them drains
    // that queue.
    constexpr bool kDqReg = !kTight && !(want_arg && !kIso && DP == 128);
    float2 dq[8];
    auto dsc_fetch = [&]() {
#pragma unroll
        for (int e = 0; e < 8; ++e) dq[e] = dsc_l[e * Sh::kCB + cbk];
    };
    // staging step s: columns 2 (s % 4), +1 of item s / 4; the item's chunks are
    // written after its fourth step
    auto stage_pair = [&](int buf, int sp) {
        const int q = sp / 4, pr = sp % 4;
        const int it = tid + NT * q;
        if (Sh::kItems % NT != 0 && it >= Sh::kItems) return;   // whole waves idle
        uint16_t* yb = ybuf[buf];
        const int r = it / Sh::kCB;
        const uint32_t wd = col_ok ? (pr == 0 ? raw[q].x : pr == 1 ? raw[q].y : pr == 2 ? raw[q].z : raw[q].w) : 0u;
        if (pr == 0) ss = 0.0f;
        float yp[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int e = 2 * pr + h;
            const float2 cs = dq[e];
            const float x = h16_to_f32<BF16>(h ? wd >> 16 : wd & 0xFFFFu);
            if constexpr (kIso) {
                const float y = col_ok ? x - cs.x : 0.0f;   // dsc_l: (c, s)
                ss = fmaf(y, y, ss);
                yp[h] = y * cs.y;
            } else {
                yp[h] = fmaf(x, cs.x, cs.y);                 // dsc_l: (s, -c s)
            }
        }
        hy[pr] = pack_h2(yp[0], yp[1]);
        if constexpr (!kIso) {
            // the square of the staged fp16 y' (one packed multiply), so the
            // score is the expanded form at the rounded point; beyond the fp16
            // range it is inf: the pass is flagged below and its results
            // are discarded
            const half2v h = __builtin_bit_cast(half2v, hy[pr]);
            const half2v q = h * h;
            rq = __builtin_elementwise_max(rq, q);
            hq[pr] = __builtin_bit_cast(uint32_t, q);
        }
        if (pr == 3) {
            const int off_y = kIso ? 0 : DP;
            *reinterpret_cast<uint4*>(yb + Sh::ych(r, (off_y + col0) / 8)) = make_uint4(hy[0], hy[1], hy[2], hy[3]);
            if constexpr (!kIso) {
                *reinterpret_cast<uint4*>(yb + Sh::ych(r, col0 / 8)) = make_uint4(hq[0], hq[1], hq[2], hq[3]);
            } else {
                // |y|^2 of the row over its kCB consecutive lanes
                float t2 = ss;
                if constexpr (Sh::kCB >= 2) t2 += dpp<kDppXor1>(t2);
                if constexpr (Sh::kCB >= 4) t2 += dpp<kDppXor2>(t2);
                if constexpr (Sh::kCB >= 8) t2 += dpp<kDppHalfMirror>(t2);
                if constexpr (Sh::kCB >= 16) t2 += dpp<kDppMirror>(t2);
                const float v = t2 * ysc;
                rng = fmaxf(rng, v);
                const float vc = fminf(v, kF16Max);
                const _Float16 yh = (_Float16)vc;
                const uint16_t hb = __builtin_bit_cast(uint16_t, yh);
                const uint16_t lb = __builtin_bit_cast(uint16_t, (_Float16)(vc - (float)yh));
                uint16_t sv[kSlots];
#pragma unroll
                for (int m = 0; m < kSlots; ++m) {
                    const int slot = kSlots * cbk + m;
                    sv[m] = slot == 0 || slot == 2 ? hb : slot == 1 ? lb : (slot == 3 || slot == 4) ? 0x3C00 : 0;
                }
                uint16_t* bp = yb + Sh::ych(r, Sh::kFCh) + kSlots * cbk;
                if constexpr (kSlots == 1) *bp = sv[0];
                else if constexpr (kSlots == 2) *reinterpret_cast<uint32_t*>(bp) = sv[0] | ((uint32_t)sv[1] << 16);
                else *reinterpret_cast<uint2*>(bp) = make_uint2(sv[0] | ((uint32_t)sv[1] << 16),
                                                                 sv[2] | ((uint32_t)sv[3] << 16));
                yh_t[buf][r] = hb;   // the kCB lanes of the row store the same value
            }
        }
    };
    auto store_tile = [&](int buf) {
        dsc_fetch();
#pragma unroll
        for (int sp = 0; sp < kPairs; ++sp) stage_pair(buf, sp);
    };

    // diagonal bias slots: constant [1, 1, 0...] in both tile buffers
    if constexpr (!kIso) {
        for (int i = tid; i < NYB * kT; i += NT) {
            uint4* bias = reinterpret_cast<uint4*>(ybuf[i / kT] + Sh::ych(i % kT, Sh::kFCh));
            bias[0] = make_uint4(0x3C003C00u, 0u, 0u, 0u);
            bias[1] = make_uint4(0u, 0u, 0u, 0u);
        }
    }

    // pipeline: tile t+1 is staged (from registers loaded during tile t-1)
    // while tile t's scores run, then tile t+2's loads are issued
    if (t0 < t1) {
        load_tile(t0);
        __syncthreads();   // dsc_l
        store_tile(0);
        load_tile(t0 + 1 < t1 ? t0 + 1 : t0);
        if constexpr (MODE == LK_SWEEP2) lse_nx = load_lse(t0);
    }
    // every prologue load (the panel above all) has landed: no wait inside the
    // tile loop depends on them
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // per-block values of the tile whose softmax is being formed
    float mcb[CB], zcb[CB];                 // per block: max (acc units), sum of exp2(F (acc - max))
    int acb[CB];                            // per block: lowest component at the max
    half2v eh[MODE == LK_FUSED_EM ? CB : 1][8];   // fused E+M: exp2(F (acc - max)), fp16 pairs

    // ---- scores of tile t from the LDS tile yb (acc units; S = F acc), one
    // 32-component block at a time: lane (pn, hf), register r of block cb
    // holds point pn and component kbase + 32 cb + 8 (r / 4) + 4 hf + r % 4;
    // tile t + 1 is staged into buffer nxt between the MFMAs and the loads of
    // tile t + 2 are issued after them
    auto score_tile = [&](int64_t t, const uint16_t* yb, int nxt, f32x16 (&scb)[CB]) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) scb[cb][r] = 0.0f;
        // operands read kPF steps ahead of their MFMAs: the tile (B, K = inner)
        // and the LDS-resident panel steps (A)
        constexpr int kPF = kTight ? 2 : 4;
        // the staging steps of the next tile, one every kSp MFMA steps (spread
        // over the whole score loop rather than its first steps: 1.5% on the
        // 2e8 x 128 x 1024 step)
        constexpr int kSp = KS / kPairs > 0 ? KS / kPairs : 1;
        constexpr auto in_lds = [](int ks) { return ks < KL || ks == KS - 1; };
        half8 yq[KS];
        half8 pq[CB][KS];
        auto issue = [&](int ks) {
            yq[ks] = *reinterpret_cast<const half8*>(yb + Sh::ych(pn, 2 * ks + hf));
            if (in_lds(ks))
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
                    pq[cb][ks] = __builtin_bit_cast(half8, plds[w][cb][ks < KL ? ks : KL][lane]);
        };
        if constexpr (!kDqReg) dsc_fetch();
#pragma unroll
        for (int ks = 0; ks < kPF && ks < KS; ++ks) issue(ks);
        // step ks: the MFMAs of step ks, then (every kSp steps) one staging step
        // of the next tile (the other buffer) while they run; the order is
        // pinned per step
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + kPF < KS) issue(ks + kPF);
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const half8 pa = in_lds(ks) ? pq[cb][ks] : pnl[cb][in_lds(ks) ? 0 : ks - KL];
                if constexpr (kAsmAcc) mfma32_v(scb[cb], pa, yq[ks], ks == 0);
                else scb[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa, yq[ks], scb[cb], 0, 0, 0);
            }
            if (ks % kSp == 0 && ks / kSp < kPairs) stage_pair(nxt, ks / kSp);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int sp = (KS + kSp - 1) / kSp; sp < kPairs; ++sp) stage_pair(nxt, sp);
        if constexpr (kAsmAcc) {
            static_assert(CB == 2, "settle both score blocks");
            mfma_v_settle(scb[0], scb[1]);
        }
        // the loads of the tile after next
        load_tile(t + 2 < t1 ? t + 2 : t1 - 1);
    };
    // ---- per block: the softmax values (modes that exchange), the slice's
    // base-2 scores (top-m) or gamma = exp2(S - lse) into LDS (sweep 2)
    auto block_phase = [&](f32x16 (&scb)[CB], uint16_t* gw, float lse_cur) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        f32x16& sc = scb[cb];
        if constexpr (kExchange) {
            float m = sc[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) m = fmaxf(m, sc[r]);
            m = halves_max(m);
            const float nmf = m == -INFINITY ? 0.0f : -F * m;
            float z = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e = fast_exp2(fmaf(sc[r], F, nmf));
                if constexpr (MODE == LK_FUSED_EM) {
                    if (r & 1) eh[cb][r >> 1] = half2v{(_Float16)sc[r - 1], (_Float16)e};
                    else sc[r] = e;
                }
                z += e;
            }
            mcb[cb] = m;
            zcb[cb] = halves_sum(z);
            acb[cb] = 0x7FFFFFFF;
            if constexpr (!kStats) {
                if (want_arg) {
                    int bi = 0x7FFFFFFF;
#pragma unroll
                    for (int r = 15; r >= 0; --r)
                        if (sc[r] == m) bi = kbase + 32 * cb + 8 * (r >> 2) + 4 * hf + (r & 3);
                    acb[cb] = halves_min(bi);
                }
            }
        } else if constexpr (kTopm) {
            // base-2 scores of the slice's components -> LDS [point][component]
#pragma unroll
            for (int r = 0; r < 16; ++r)
                stile[pn][w * KW + 32 * cb + 8 * (r >> 2) + 4 * hf + (r & 3)] = F * sc[r];
        } else {
            // sweep 2: gamma = exp2(S - lse) (lse = +inf beyond N) -> LDS [point][component]
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float gv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) gv[e] = fast_exp2(fmaf(sc[4 * q + e], F, -lse_cur));
                *reinterpret_cast<uint2*>(gw + gch<KW>(pn, 8 * cb + 2 * q + hf)) =
                    make_uint2(pack_h2(gv[0], gv[1]), pack_h2(gv[2], gv[3]));
            }
        }
    }
    };
    // ---- this wave's (max, sum) per point into exchange buffer par
    auto wave_part = [&](int par) {
        float2(*wpart)[kT] = wpart_b[kOneBarrier ? par : 0];
        int(*warg)[kT] = warg_b[kOneBarrier ? par : 0];
        // this wave's (max, sum) per point, base-2 score units
        float m = mcb[0];
#pragma unroll
        for (int cb = 1; cb < CB; ++cb) m = fmaxf(m, mcb[cb]);
        const float Fm = m == -INFINITY ? -INFINITY : F * m;
        float z = 0.0f;
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int cb = CB - 1; cb >= 0; --cb) {
            if (mcb[cb] != -INFINITY) z = fmaf(zcb[cb], fast_exp2(F * (mcb[cb] - m)), z);
            if (mcb[cb] == m) bi = acb[cb];
        }
        if (hf == 0) {
            wpart[w][pn] = make_float2(Fm, z);
            if (want_arg) warg[w][pn] = bi;
        }
    };
    // ---- after the exchange barrier: the LSE (and argmax) over the slice of
    // the points of tile t from exchange buffer par, and what the mode writes
    // (lanes of the lower half of wave `owner` write the per-point values)
    auto combine = [&](int64_t t, int par, uint16_t* gw, bool owner) {
        float2(*wpart)[kT] = wpart_b[kOneBarrier ? par : 0];
        int(*warg)[kT] = warg_b[kOneBarrier ? par : 0];
        const int64_t prow = t * kT;
        const bool pvalid = prow + pn < n;
        // the waves of this wave's slice: w0 .. w0 + WV - 1
        float M = wpart[w0][pn].x;
#pragma unroll
        for (int w2 = 1; w2 < WV; ++w2) M = fmaxf(M, wpart[w0 + w2][pn].x);
        const float Ms = M == -INFINITY ? 0.0f : M;
        float Z = 0.0f;
#pragma unroll
        for (int w2 = 0; w2 < WV; ++w2) {
            const float2 mz = wpart[w0 + w2][pn];
            Z = fmaf(mz.y, fast_exp2(mz.x - Ms), Z);
        }
        float lse = Ms + fast_log2(Z);
        int arg = 0;
        if (want_arg) {
            arg = 0x7FFFFFFF;
#pragma unroll
            for (int w2 = WV - 1; w2 >= 0; --w2)
                if (wpart[w0 + w2][pn].x == M) arg = warg[w0 + w2][pn];
        }
        const int64_t p = prow + pn;
        if constexpr (MODE == LK_FUSED_EM || MODE == LK_FUSED_E) {
            if (nxc > 0 && pvalid) {   // merge the exactly scored components
                const float xl = a.xlse[p];
                const float m2 = fmaxf(lse, xl);
                if (m2 != -INFINITY) lse = m2 + fast_log2(fast_exp2(lse - m2) + fast_exp2(xl - m2));
                if constexpr (MODE == LK_FUSED_E) {
                    if (want_arg) {
                        const float xm = a.xmax[p];
                        const int xa = a.xarg[p];
                        if (xm > M || (xm == M && xa < arg)) arg = xa;
                    }
                } else if (owner && hf == 0) {
                    a.lse_out[p] = lse;   // their statistics pass reads it
                }
            }
        }
        if (owner && hf == 0 && pvalid) {
            if constexpr (MODE == LK_SWEEP1) {
                a.part_lse[(int64_t)slice * n + p] = lse;
                if (want_arg) {
                    a.part_arg[(int64_t)slice * n + p] = arg;
                    a.part_max[(int64_t)slice * n + p] = M;
                }
            } else {
                ll2 += (double)lse;
                if constexpr (MODE == LK_FUSED_E) {
                    if (a.out_lse) a.out_lse[p] = lse * kLn2f;
                    if (want_arg) a.out_arg[p] = arg;
                }
            }
        }
        if constexpr (MODE == LK_FUSED_EM) {
            // gamma = exp2(F (acc - m_cb)) exp2(F m_cb - lse), zero beyond N -> LDS
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const float f = (pvalid && mcb[cb] != -INFINITY) ? fast_exp2(F * mcb[cb] - lse) : 0.0f;
                const half2v f2 = {(_Float16)f, (_Float16)f};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const half2v g0 = eh[cb][2 * q] * f2, g1 = eh[cb][2 * q + 1] * f2;
                    *reinterpret_cast<uint2*>(gw + gch<KW>(pn, 8 * cb + 2 * q + hf)) =
                        make_uint2(__builtin_bit_cast(uint32_t, g0), __builtin_bit_cast(uint32_t, g1));
                }
            }
        }
    };

    if constexpr (SPW == 2 && !want_arg) {
        // Two slices per workgroup, one wave of each on every SIMD: the
        // second slice's waves run half a tile behind the first's.  Between
        // two barriers the first slice scores tile t and forms its softmax;
        // the second forms the softmax of tile t - 1 (its scores kept in
        // registers across the barrier) and then scores tile t.  Each slice
        // combines the exchange of its previous tile after the barrier.  On
        // a 2e8 x 128 x 1024 step this measured about 1% faster than both
        // slices in step.  (Not in the argmax variants, whose registers it
        // would overflow at D = 128.)
        const bool lag = w >= WV;
        f32x16 scb[CB];
        for (int64_t t = t0; t < t1; ++t) {
            const int cur = (int)((t - t0) & 1), par = cur;
            if (t > t0 && (!lag || t - 1 > t0)) combine(lag ? t - 2 : t - 1, par ^ 1, nullptr, wl == 0);
            if (!lag) {
                score_tile(t, ybuf[cur], cur ^ 1, scb);
                block_phase(scb, nullptr, 0.0f);
                wave_part(par);
            } else {
                if (t > t0) {
                    block_phase(scb, nullptr, 0.0f);
                    wave_part(par);
                }
                score_tile(t, ybuf[cur], cur ^ 1, scb);
            }
            __syncthreads();
        }
        if (t0 < t1) {
            const int par = (int)((t1 - t0) & 1);
            if (!lag || t1 - 1 > t0) combine(lag ? t1 - 2 : t1 - 1, par ^ 1, nullptr, wl == 0);
            if (lag) {
                block_phase(scb, nullptr, 0.0f);
                wave_part(par);
            }
            __syncthreads();
            if (lag) combine(t1 - 1, par, nullptr, wl == 0);
        }
    } else {
        for (int64_t t = t0; t < t1; ++t) {
            const int cur = (int)((t - t0) % NYB), nxt = cur + 1 == NYB ? 0 : cur + 1;
            const int par = (int)((t - t0) & 1);
            const uint16_t* yb = ybuf[cur];
            const int64_t prow = t * kT;
            float lse_cur = 0.0f;
            if constexpr (MODE == LK_SWEEP2) {
                lse_cur = lse_nx;
                lse_nx = load_lse(t + 1 < t1 ? t + 1 : t);
            }
            uint16_t* gw = gbuf[kStats ? w : 0];
            f32x16 scb[CB];
            score_tile(t, yb, nxt, scb);
            block_phase(scb, gw, lse_cur);
            if constexpr (kExchange) {
                wave_part(par);
                __syncthreads();
                combine(t, par, gw, wl == 0);
            }

            if constexpr (kTopm) {
                __syncthreads();   // the tile's scores are in stile
                topm_tile(prow);
            }

            // ---- statistics MFMAs from the responsibility tile (wave-private)
            if constexpr (kStats) {
                // A operands: gamma^T (row = component, K = 16 points per step);
                // B operands: the tile of X (K = points, column = feature), read
                // two feature blocks ahead of their MFMAs
                constexpr int kSteps = 2 * NFB;                 // (kp, fb)
                constexpr int kPFB = kTight ? 1 : 2;
                half8 bzq[kSteps];
                half8 ag[2][CB];
                // transposed reads: lane i of 16-lane group q takes row 16 kp + 8 (q / 2) + i / 4 (+ 4)
                const int trow = 8 * (gq >> 1) + (gi >> 2);
                auto bz_read = [&](int i) {
                    const int kp = i / NFB, fb = i % NFB;
                    const int r = 16 * kp + trow, c = 4 * fb + 2 * (gq & 1) + ((gi & 3) >> 1), o = 4 * (gi & 1);
                    const uint2 lo = tr16(yb + Sh::ych(r, c) + o), hi = tr16(yb + Sh::ych(r + 4, c) + o);
                    return __builtin_bit_cast(half8, make_uint4(lo.x, lo.y, hi.x, hi.y));
                };
                auto g_read = [&](int r, int u) {
                    const uint2 lo = tr16(gw + gch<KW>(r, u)), hi = tr16(gw + gch<KW>(r + 4, u));
                    return __builtin_bit_cast(half8, make_uint4(lo.x, lo.y, hi.x, hi.y));
                };
#pragma unroll
                for (int kp = 0; kp < 2; ++kp)
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb)
                        ag[kp][cb] = g_read(16 * kp + trow, 8 * cb + 4 * (gq & 1) + (gi & 3));
#pragma unroll
                for (int i = 0; i < kPFB; ++i) bzq[i] = bz_read(i);
#pragma unroll
                for (int i = 0; i < kSteps; ++i) {
                    if (i + kPFB < kSteps) bzq[i + kPFB] = bz_read(i + kPFB);
                    const int kp = i / NFB, fb = i % NFB;
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb)
                        acc[cb][fb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ag[kp][cb], bzq[i], acc[cb][fb], 0, 0, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x100, 2 * (2 * CB + kPFB), 1);
#pragma unroll
                for (int i = 0; i < kSteps; ++i) {
                    if (i + kPFB < kSteps) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
                    __builtin_amdgcn_sched_group_barrier(0x008, CB, 1);
                }
                // s0 (and iso sum gamma |y|^2): 16 components x 32 points against [1, yh]
                half8 bx;
                {
                    const uint4 hv = *reinterpret_cast<const uint4*>(&yh_t[cur][8 * gq]);
                    const uint4 ones = make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);
                    const uint4 z4 = make_uint4(0, 0, 0, 0);
                    bx = __builtin_bit_cast(half8, gi == 0 ? ones : ((kIso && gi == 1) ? hv : z4));
                }
#pragma unroll
                for (int b = 0; b < KW / 16; ++b) {
                    const half8 ax = g_read(8 * gq + (gi >> 2), 4 * b + (gi & 3));
                    if constexpr (kAsmAcc) mfma16_v(aux[b], ax, bx);
                    else aux[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ax, bx, aux[b], 0, 0, 0);
                }
            }

            // one-barrier modes: the next tile was staged by every wave before the
            // exchange barrier, and the tile staged during the next one is not
            // this one (three buffers when the statistics read this tile after it)
            if constexpr (!kOneBarrier) __syncthreads();
        }
    }

    if constexpr (kAsmAcc) {
        static_assert(KW / 16 == 4, "settle the s0 accumulators");
        mfma_v_settle(aux[0], aux[1], aux[2], aux[3]);
    }
    // ---- epilogue: per-workgroup partials, one writer per value
    if constexpr (!kIso) rng = fmaxf((float)rq[0], (float)rq[1]);
    const int flag = __syncthreads_or(rng > kF16Max ? 1 : 0);
    const bool first = a.seg_first != 0;
    if (tid == 0) a.part_flag[blockIdx.x] = first ? flag : (a.part_flag[blockIdx.x] | flag);
    if constexpr (kStats) {
        const int ncol = kIso ? 2 + d : 1 + 2 * d;
        double* dst = a.part + (int64_t)blockIdx.x * kLkSlice * ncol;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int fb = 0; fb < NFB; ++fb) {
                const int f = 32 * fb + pn;
                int col = -1;
                if (kIso) col = f < d ? 1 + f : -1;
                else if (f < DP) col = f < d ? 1 + d + f : -1;          // y'^2 -> s2'
                else col = f - DP < d ? 1 + (f - DP) : -1;              // y'   -> s1'
                if (col >= 0) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int kl = w * KW + 32 * cb + 8 * (r >> 2) + 4 * hf + (r & 3);
                        double* o = dst + (int64_t)kl * ncol + col;
                        *o = first ? (double)acc[cb][fb][r] : *o + (double)acc[cb][fb][r];
                    }
                }
            }
        if (gi < (kIso ? 2 : 1)) {
            const double scl = gi == 0 ? 1.0 : (double)a.prm[2];   // iso: undo the 2^-g of yh
#pragma unroll
            for (int b = 0; b < KW / 16; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int kl = w * KW + 16 * b + 4 * gq + r;
                    double* o = dst + (int64_t)kl * ncol + (gi == 0 ? 0 : 1 + d);
                    *o = first ? (double)aux[b][r] * scl : *o + (double)aux[b][r] * scl;
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
        if (tid == 0) a.part_ll[blockIdx.x] = first ? llred[0] * kLn2 : a.part_ll[blockIdx.x] + llred[0] * kLn2;
    }
}

template <int COV, int DP, int MODE, bool VEC>
hipError_t launch4(const Plan& p, const LkArgs& a, int grid, hipStream_t s) {
    if (p.xdt == GMM_BF16)
        hipLaunchKernelGGL((k_lk<COV, DP, MODE, true, VEC>), dim3(grid), dim3(lk_threads(MODE, COV)), 0, s, a);
    else
        hipLaunchKernelGGL((k_lk<COV, DP, MODE, false, VEC>), dim3(grid), dim3(lk_threads(MODE, COV)), 0, s, a);
    return hipGetLastError();
}

template <int COV, int DP, int MODE>
hipError_t launch3(const Plan& p, const LkArgs& a, int grid, hipStream_t s) {
    return a.vec ? launch4<COV, DP, MODE, true>(p, a, grid, s) : launch4<COV, DP, MODE, false>(p, a, grid, s);
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
        case LK_SWEEP1 | kLkArg: return launch2<COV, LK_SWEEP1 | kLkArg>(p, a, grid, s);
        case LK_SWEEP1 | kLkPair: return launch2<COV, LK_SWEEP1 | kLkPair>(p, a, grid, s);
        case LK_SWEEP1 | kLkArg | kLkPair: return launch2<COV, LK_SWEEP1 | kLkArg | kLkPair>(p, a, grid, s);
        case LK_SWEEP2: return launch2<COV, LK_SWEEP2>(p, a, grid, s);
        case LK_FUSED_E: return launch2<COV, LK_FUSED_E>(p, a, grid, s);
        case LK_FUSED_E | kLkArg: return launch2<COV, LK_FUSED_E | kLkArg>(p, a, grid, s);
        case LK_TOPM: return launch2<COV, LK_TOPM>(p, a, grid, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t lk_launch(const Plan& p, const LkArgs& a, int mode, int grid, hipStream_t s) {
    // the argmax variants when the caller asked for it
    const bool arg = (mode == LK_SWEEP1 && a.part_arg != nullptr) || (mode == LK_FUSED_E && a.out_arg != nullptr);
    mode = lk_plan_mode(p, mode);
    if (arg) mode |= kLkArg;
    if (p.cov == GMM_COV_ISO) return launch1<GMM_COV_ISO>(p, a, mode, grid, s);
    return launch1<GMM_COV_DIAG>(p, a, mode, grid, s);
}

}  // namespace gmm
