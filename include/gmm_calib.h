/*
 * gmm_calib.h - calibration kernels of libgmm: measured ceilings of the
 * device, reported beside the published peaks when a kernel is priced
 * against its roofline.
 *
 * Source: the operator-debugging toolkit article (2kiu.com/news/5842513),
 * section 4.1 (a kernel's lower bound from its bytes and flops) and section
 * 6.2 (a calibration operator run on the same machine to normalise the
 * measurement).  They are measurement infrastructure, not part of the EM
 * iteration.  Conventions as in gmm.h: device pointers, caller-owned
 * buffers, asynchronous on `stream`, no allocation.
 */
#ifndef GMM_CALIB_H
#define GMM_CALIB_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "gmm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of the device `sink` buffer both calibration kernels need for a grid
 * of `grid` workgroups (one 4-byte value per thread). */
size_t gmm_calib_sink_bytes(int grid);

/* Streaming read: every 16-byte vector of `buf` (device, 16-byte aligned,
 * `bytes` >= 16, the tail beyond a multiple of 16 is ignored) is loaded once
 * by a grid-stride loop of `grid` workgroups; a digest per thread goes to
 * `sink`.  Achieved bandwidth = (bytes / 16 * 16) / elapsed time.
 * GMM_E_ARG on a null or misaligned pointer or grid < 1. */
gmm_status gmm_calib_read(const void* buf, size_t bytes, int grid, void* sink,
                          hipStream_t stream);

/* Matrix-core ceiling: `grid` workgroups of four waves, each issuing `iters`
 * x 4 independent v_mfma_f32_32x32x16_f16 from registers (no memory traffic
 * in the loop); the sums go to `sink`.  GMM_E_ARG on iters < 1, grid < 1. */
gmm_status gmm_calib_mfma(int64_t iters, int grid, void* sink, hipStream_t stream);

/* Floating-point operations gmm_calib_mfma(iters, grid, ...) performs. */
double gmm_calib_mfma_flops(int64_t iters, int grid);

#ifdef __cplusplus
}
#endif

#endif /* GMM_CALIB_H */
