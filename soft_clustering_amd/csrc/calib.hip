// Calibration kernels: the machine's own ceilings, measured, for the
// denominators that sit beside the published peaks.  The operator-debugging
// article prices a kernel against a lower bound from its bytes and flops
// (section 4.1) and normalises for the machine with a calibration operator
// (section 6.2); these are those operators for HBM and the fp16 matrix cores.
//
//   k_calib_read  - streaming read of a caller buffer (16-byte loads, grid
//                   stride), every byte read once, one value written per thread;
//   k_calib_mfma  - register-resident chains of v_mfma_f32_32x32x16_f16 (the
//                   instruction the large-K kernels use), no memory traffic in
//                   the loop, one value written per lane.

#include "common.h"
#include "gmm_calib.h"

namespace gmm {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kCalibThreads = 256;
constexpr int kCalibChains = 4;   // independent accumulator chains per wave

__global__ __launch_bounds__(kCalibThreads) void k_calib_read(const uint4* __restrict__ buf,
                                                              int64_t nvec, uint32_t* __restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * kCalibThreads;
    uint32_t a0 = 0, a1 = 0;
    int64_t i = (int64_t)blockIdx.x * kCalibThreads + threadIdx.x;
    // two loads in flight per iteration per lane
    for (; i + stride < nvec; i += 2 * stride) {
        const uint4 v = buf[i], u = buf[i + stride];
        a0 ^= v.x ^ v.y ^ v.z ^ v.w;
        a1 ^= u.x ^ u.y ^ u.z ^ u.w;
    }
    if (i < nvec) {
        const uint4 v = buf[i];
        a0 ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    sink[(int64_t)blockIdx.x * kCalibThreads + threadIdx.x] = a0 ^ a1;
}

__global__ __launch_bounds__(kCalibThreads) void k_calib_mfma(int64_t iters, float seed,
                                                              float* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const _Float16 h = (_Float16)(seed * (float)(lane + 1));
    const half8 a = {h, h, h, h, h, h, h, h};
    const half8 b = {(_Float16)1.0f, (_Float16)0.5f, (_Float16)0.25f, (_Float16)0.125f,
                     (_Float16)1.0f, (_Float16)0.5f, (_Float16)0.25f, (_Float16)0.125f};
    f32x16 acc[kCalibChains];
#pragma unroll
    for (int c = 0; c < kCalibChains; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kCalibChains; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kCalibChains; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    sink[(int64_t)blockIdx.x * kCalibThreads + threadIdx.x] = s;
}

}  // namespace

}  // namespace gmm

using namespace gmm;

extern "C" {

size_t gmm_calib_sink_bytes(int grid) {
    return grid > 0 ? sizeof(uint32_t) * (size_t)grid * kCalibThreads : 0;
}

gmm_status gmm_calib_read(const void* buf, size_t bytes, int grid, void* sink, hipStream_t stream) {
    if (buf == nullptr || sink == nullptr || grid < 1 || bytes < 16) return GMM_E_ARG;
    if ((uintptr_t)buf % 16 != 0) return GMM_E_ARG;
    hipLaunchKernelGGL(k_calib_read, dim3(grid), dim3(kCalibThreads), 0, stream,
                       (const uint4*)buf, (int64_t)(bytes / 16), (uint32_t*)sink);
    return hipGetLastError() == hipSuccess ? GMM_OK : GMM_E_HIP;
}

gmm_status gmm_calib_mfma(int64_t iters, int grid, void* sink, hipStream_t stream) {
    if (sink == nullptr || grid < 1 || iters < 1) return GMM_E_ARG;
    hipLaunchKernelGGL(k_calib_mfma, dim3(grid), dim3(kCalibThreads), 0, stream, iters, 1.0e-3f,
                       (float*)sink);
    return hipGetLastError() == hipSuccess ? GMM_OK : GMM_E_HIP;
}

double gmm_calib_mfma_flops(int64_t iters, int grid) {
    // per wave and iteration: kCalibChains instructions of 2 * 32 * 32 * 16 flops
    return (double)grid * (kCalibThreads / 64) * (double)iters * kCalibChains * 2.0 * 32 * 32 * 16;
}

}  // extern "C"
