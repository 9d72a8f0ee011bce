// Device helpers shared by the libgmm kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gmm {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr double kLog2e = 1.4426950408889634074;
constexpr double kLn2 = 0.69314718055994530942;
constexpr double kLog2Pi = 1.8378770664093454836;   // natural log of 2*pi
constexpr double kEmptyNk = 1e-6;                   // s0 below this: empty component

// Lane l of a wave64 is (g, j) = (l / 16, l % 16).  For v_mfma_f32_16x16x4f32
// the A operand of lane l is A[j][g], the B operand is B[g][j], and the four
// accumulator registers hold D[4g + r][j], r = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Butterfly over one 16-lane DPP row: swap neighbours, swap pairs, mirror
// the half-rows, mirror the row.  Every pairing is symmetric, so all 16
// lanes end with bitwise the same result (a+b == b+a).
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror
constexpr int kDppMirror = 0x140;      // row_mirror

__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp<kDppXor1>(v));
    v = fmaxf(v, dpp<kDppXor2>(v));
    v = fmaxf(v, dpp<kDppHalfMirror>(v));
    v = fmaxf(v, dpp<kDppMirror>(v));
    return v;
}

__device__ __forceinline__ float row16_sum(float v) {
    v = v + dpp<kDppXor1>(v);
    v = v + dpp<kDppXor2>(v);
    v = v + dpp<kDppHalfMirror>(v);
    v = v + dpp<kDppMirror>(v);
    return v;
}

__device__ __forceinline__ int row16_min_i(int v) {
    v = min(v, __builtin_amdgcn_update_dpp(0, v, kDppXor1, 0xF, 0xF, false));
    v = min(v, __builtin_amdgcn_update_dpp(0, v, kDppXor2, 0xF, 0xF, false));
    v = min(v, __builtin_amdgcn_update_dpp(0, v, kDppHalfMirror, 0xF, 0xF, false));
    v = min(v, __builtin_amdgcn_update_dpp(0, v, kDppMirror, 0xF, 0xF, false));
    return v;
}

// Hardware base-2 transcendental instructions (v_exp_f32, v_log_f32).
// The values of v in lanes l and l ^ 32 (the two halves of a wave of 64)
// from one v_permlane32_swap, a VALU exchange (a shuffle is an LDS round
// trip, which also waits for every LDS access issued before it).  In every
// lane .x is the lower half's value and .y the upper half's, so combining
// the two gives bitwise the same result in both lanes.
__device__ __forceinline__ uint2 wave_halves(uint32_t v) {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return make_uint2(r[0], r[1]);
}
__device__ __forceinline__ float halves_max(float v) {
    const uint2 h = wave_halves(__float_as_uint(v));
    return fmaxf(__uint_as_float(h.x), __uint_as_float(h.y));
}
__device__ __forceinline__ float halves_sum(float v) {
    const uint2 h = wave_halves(__float_as_uint(v));
    return __uint_as_float(h.x) + __uint_as_float(h.y);
}
__device__ __forceinline__ int halves_min(int v) {
    const uint2 h = wave_halves((uint32_t)v);
    return min((int)h.x, (int)h.y);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Storage types of X.
struct bf16_t { uint16_t bits; };

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return __uint_as_float(((uint32_t)v.bits) << 16); }
__device__ __forceinline__ float to_f32(_Float16 v) { return (float)v; }

// Unpack a 16-byte vector of storage elements into fp32.
template <typename XT> struct Vec16;
template <> struct Vec16<float> {
    static constexpr int kElems = 4;
    __device__ __forceinline__ static void unpack(const uint4& v, float* o) {
        o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
        o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
    }
};
template <> struct Vec16<bf16_t> {
    static constexpr int kElems = 8;
    __device__ __forceinline__ static void unpack(const uint4& v, float* o) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = __uint_as_float(w[i] << 16);
            o[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    }
};
template <> struct Vec16<_Float16> {
    static constexpr int kElems = 8;
    __device__ __forceinline__ static void unpack(const uint4& v, float* o) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            _Float16 lo, hi;
            uint16_t l16 = (uint16_t)(w[i] & 0xFFFF), h16 = (uint16_t)(w[i] >> 16);
            __builtin_memcpy(&lo, &l16, 2);
            __builtin_memcpy(&hi, &h16, 2);
            o[2 * i] = (float)lo;
            o[2 * i + 1] = (float)hi;
        }
    }
};

// Device-side health counters (mirrors gmm_diag, minus the LL).
struct DevDiag {
    int bad_params;
    int not_pd;
    int ridge_retries;
    int empty;
    int nonfinite;
    int reserved;
};

// Deterministic block-wide sum of one double per thread (fixed tree order).
// `scratch` must hold blockDim.x doubles; all threads must call it.
__device__ __forceinline__ double block_sum_f64(double v, double* scratch) {
    const int t = threadIdx.x;
    scratch[t] = v;
    __syncthreads();
    for (int s = blockDim.x / 2; s > 0; s >>= 1) {
        if (t < s) scratch[t] += scratch[t + s];
        __syncthreads();
    }
    double r = scratch[0];
    __syncthreads();
    return r;
}

}  // namespace gmm
