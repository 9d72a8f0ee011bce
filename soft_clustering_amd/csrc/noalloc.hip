// One EM iteration that allocates nothing and takes no workspace: for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation).  The workspace is a
// fixed-size file-scope device array; each device holds its own copy for the
// life of the process.  Every call on a device shares that device's copy, so
// calls that overlap on one device race.  The call runs gmm_prepare (which
// resets every flag and counter the kernels rely on), gmm_em_step and
// gmm_finalize on it, exactly as a caller-owned workspace would.

#include <mutex>

#include "common.h"
#include "plan.h"

namespace gmm {

namespace {

constexpr size_t kScratchBytes = (size_t)128 << 20;   // the largest plan it serves
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {nullptr};

// This device's address of `scratch` (the host-side name is only a stand-in),
// looked up once per device with the device current.
gmm_status scratch_ptr(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GMM_E_HIP;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return GMM_E_HIP;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return GMM_OK;
}

}  // namespace

}  // namespace gmm

using namespace gmm;

extern "C" {

gmm_status gmm_prepare(const gmm_desc*, void*, size_t, const float*, const float*, const float*,
                       hipStream_t);
gmm_status gmm_em_step(const gmm_desc*, void*, size_t, const void*, double*, hipStream_t);
gmm_status gmm_finalize(const gmm_desc*, void*, size_t, float*, float*, float*, hipStream_t);

size_t gmm_noalloc_max_workspace(void) { return kScratchBytes; }

gmm_status gmm_em_iteration_noalloc(const gmm_desc* desc, const float* pi, const float* mu,
                                    const float* cov, const void* x, double* ll_out,
                                    float* pi_out, float* mu_out, float* cov_out,
                                    hipStream_t stream) {
    Plan p;
    gmm_status st = make_plan(desc, &p);
    if (st != GMM_OK) return st;
    if (p.total > kScratchBytes) return GMM_E_WORKSPACE;
    void* ws = nullptr;
    if ((st = scratch_ptr(&ws)) != GMM_OK) return st;
    if ((st = gmm_prepare(desc, ws, kScratchBytes, pi, mu, cov, stream)) != GMM_OK) return st;
    if ((st = gmm_em_step(desc, ws, kScratchBytes, x, ll_out, stream)) != GMM_OK) return st;
    return gmm_finalize(desc, ws, kScratchBytes, pi_out, mu_out, cov_out, stream);
}

}  // extern "C"
