// EM to convergence: the seeded random-points start, and the loop of
// gmm_em_step + gmm_finalize with a log-likelihood tolerance ([Flash-GMM]
// Method, outputs: the fused step is called repeatedly until the
// log-likelihood converges; [LP-GMM] 1.1: training repeats E and M steps).
//
// One iteration = em_step (LL of theta_t, statistics) -> finalize (theta_t+1,
// and the workspace prepared for it) -> k_fit_check -> k_fit_commit.  The
// iteration is captured once into a HIP graph and replayed in batches; the host
// synchronises once per batch to read the stop flag.  Iterations replayed
// after the device decided to stop change nothing the caller sees: the check
// kernel no longer records, and the commit kernel no longer copies theta into
// the caller's buffers.
//
// Start (gmm_fit_opts.init = GMM_INIT_RANDOM_POINTS): K distinct rows of X by
// Floyd's K-subset algorithm (Bentley and Floyd, "A sample of brilliance",
// CACM 1987) drawn from SplitMix64 (Steele, Lea and Flood, OOPSLA 2014; the
// 64-bit form with the golden-ratio increment and the variant-13 output
// mixer), the draw in [0, j] being the output modulo j + 1; the rows in
// increasing index order become the means, with unit (co)variances and weights
// 1/K.

#include <algorithm>
#include <math.h>
#include <string.h>

#include "common.h"
#include "plan.h"

namespace gmm {

namespace {

struct FitCtl {
    int stop;        // 1: no further iteration is recorded or committed
    int iter;        // iterations recorded
    int max_iter;
    int copy;        // the current iteration's theta is committed
    int nonfinite;   // stopped on a non-finite LL
    int pad;
    double ll_prev;  // LL of the previous iteration
    double tol_n;    // tol * N
};
static_assert(sizeof(FitCtl) <= 64, "control block");

__global__ void k_fit_reset(FitCtl* c, int max_iter, double tol_n) {
    c->stop = 0;
    c->iter = 0;
    c->max_iter = max_iter;
    c->copy = 0;
    c->nonfinite = 0;
    c->pad = 0;
    c->ll_prev = 0.0;
    c->tol_n = tol_n;
}

// One thread: record LL(theta_t), decide whether theta_t+1 (already in the
// workspace) is committed and whether the loop stops.
__global__ void k_fit_check(FitCtl* c, const double* ll_ws, double* ll_hist) {
    if (c->stop) {
        c->copy = 0;
        return;
    }
    const int it = c->iter;
    const double ll = *ll_ws;
    if (ll_hist != nullptr) ll_hist[it] = ll;
    c->iter = it + 1;
    if (!isfinite(ll)) {   // theta_t+1 would come from non-finite statistics
        c->stop = 1;
        c->nonfinite = 1;
        c->copy = 0;
        return;
    }
    c->copy = 1;
    const bool conv = it >= 1 && fabs(ll - c->ll_prev) < c->tol_n;
    c->ll_prev = ll;
    if (conv || it + 1 >= c->max_iter) c->stop = 1;
}

// Copy the workspace theta (pi [K], mu [K*D], cov) to the caller when the
// check committed this iteration.
__global__ __launch_bounds__(256) void k_fit_commit(const FitCtl* c, const float* __restrict__ th_pi,
                                                    const float* __restrict__ th_mu,
                                                    const float* __restrict__ th_cov, int64_t n_pi,
                                                    int64_t n_mu, int64_t n_cov, float* pi, float* mu,
                                                    float* cov) {
    if (!c->copy) return;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_pi + n_mu + n_cov; i += stride) {
        if (i < n_pi) pi[i] = th_pi[i];
        else if (i < n_pi + n_mu) mu[i - n_pi] = th_mu[i - n_pi];
        else cov[i - n_pi - n_mu] = th_cov[i - n_pi - n_mu];
    }
}

// The random-points start: mu_k = x[idx_k] (fp32 of the stored value),
// unit (co)variances, pi = 1/K.  Grid K, 128 threads.
template <typename XT>
__global__ __launch_bounds__(128) void k_fit_start(const XT* __restrict__ x, int64_t ldx, int d,
                                                   int k_real, int cov_type, const int64_t* idx,
                                                   float* pi, float* mu, float* cov) {
    const int k = blockIdx.x;
    const int64_t row = idx[k];
    for (int dd = threadIdx.x; dd < d; dd += blockDim.x) {
        mu[(int64_t)k * d + dd] = to_f32(x[row * ldx + dd]);
        if (cov_type == GMM_COV_DIAG) cov[(int64_t)k * d + dd] = 1.0f;
        if (cov_type == GMM_COV_FULL)
            for (int c = 0; c < d; ++c) cov[((int64_t)k * d + dd) * d + c] = dd == c ? 1.0f : 0.0f;
    }
    if (threadIdx.x == 0) {
        pi[k] = 1.0f / (float)k_real;
        if (cov_type == GMM_COV_ISO) cov[k] = 1.0f;
    }
}

uint64_t splitmix64_next(uint64_t& s) {
    s += 0x9E3779B97F4A7C15ull;
    uint64_t z = s;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

constexpr int kMaxStartK = 4096;   // the largest K of any plan

// K distinct indices of [0, n) by Floyd's algorithm, sorted; an open-address
// set on the stack (no allocation).
void floyd_sample(int64_t n, int k, uint64_t seed, int64_t* out) {
    constexpr int kSlots = 2 * kMaxStartK;
    int64_t set[kSlots];
    for (int i = 0; i < kSlots; ++i) set[i] = -1;
    auto slot = [&](int64_t v) {
        uint32_t h = (uint32_t)(((uint64_t)v * 0x9E3779B97F4A7C15ull) >> 51) % kSlots;
        while (set[h] != -1 && set[h] != v) h = (h + 1) % kSlots;
        return h;
    };
    uint64_t s = seed;
    int m = 0;
    for (int64_t j = n - k; j < n; ++j) {
        const int64_t t = (int64_t)(splitmix64_next(s) % (uint64_t)(j + 1));
        const uint32_t ht = slot(t);
        const int64_t v = set[ht] == t ? j : t;
        set[slot(v)] = v;
        out[m++] = v;
    }
    std::sort(out, out + m);
}

size_t theta_cov_elems(const Plan& p) {
    if (p.cov == GMM_COV_ISO) return (size_t)p.k;
    if (p.cov == GMM_COV_FULL) return (size_t)p.k * p.d * p.d;
    return (size_t)p.k * p.d;
}

}  // namespace

// Workspace bytes of the fit control block and the start's indices.
size_t fit_ctl_bytes(const Plan& p) { return 64 + sizeof(int64_t) * (size_t)p.k; }

}  // namespace gmm

using namespace gmm;

extern "C" {

gmm_status gmm_em_step(const gmm_desc*, void*, size_t, const void*, double*, hipStream_t);
gmm_status gmm_finalize(const gmm_desc*, void*, size_t, float*, float*, float*, hipStream_t);
gmm_status gmm_prepare(const gmm_desc*, void*, size_t, const float*, const float*, const float*,
                       hipStream_t);

gmm_status gmm_fit(const gmm_desc* desc, void* ws, size_t ws_bytes, const void* x,
                   const gmm_fit_opts* opts, float* pi, float* mu, float* cov, double* ll_hist,
                   int32_t* n_iter, hipStream_t stream) {
    Plan p;
    gmm_status st = make_plan(desc, &p);
    if (st != GMM_OK) return st;
    if (ws == nullptr || (uintptr_t)ws % 256 != 0) return GMM_E_ARG;
    if (ws_bytes < p.total) return GMM_E_WORKSPACE;
    if (opts == nullptr || x == nullptr || pi == nullptr || mu == nullptr || cov == nullptr) return GMM_E_ARG;
    if (opts->max_iter < 1 || opts->batch < 1 || !(opts->tol >= 0.0) || !isfinite(opts->tol))
        return GMM_E_ARG;
    if (opts->init != GMM_INIT_GIVEN && opts->init != GMM_INIT_RANDOM_POINTS) return GMM_E_ARG;
    if (p.n < 1) return GMM_E_ARG;
    char* base = (char*)ws;
    FitCtl* ctl = (FitCtl*)(base + p.off_ctl);
    int64_t* start_idx = (int64_t*)(base + p.off_ctl + 64);

    // ---- start
    if (hipStreamSynchronize(stream) != hipSuccess) return GMM_E_HIP;
    if (opts->init == GMM_INIT_RANDOM_POINTS) {
        if (p.k > p.n || p.k > kMaxStartK) return GMM_E_ARG;
        int64_t idx[kMaxStartK];
        floyd_sample(p.n, (int)p.k, opts->seed, idx);
        if (hipMemcpy(start_idx, idx, sizeof(int64_t) * p.k, hipMemcpyHostToDevice) != hipSuccess)
            return GMM_E_HIP;
        switch (p.xdt) {
            case GMM_F32:
                hipLaunchKernelGGL(k_fit_start<float>, dim3(p.k), dim3(128), 0, stream, (const float*)x, p.ldx,
                                   (int)p.d, (int)p.k, p.cov, start_idx, pi, mu, cov);
                break;
            case GMM_BF16:
                hipLaunchKernelGGL(k_fit_start<bf16_t>, dim3(p.k), dim3(128), 0, stream, (const bf16_t*)x,
                                   p.ldx, (int)p.d, (int)p.k, p.cov, start_idx, pi, mu, cov);
                break;
            default:
                hipLaunchKernelGGL(k_fit_start<_Float16>, dim3(p.k), dim3(128), 0, stream,
                                   (const _Float16*)x, p.ldx, (int)p.d, (int)p.k, p.cov, start_idx, pi,
                                   mu, cov);
        }
        if (hipGetLastError() != hipSuccess) return GMM_E_HIP;
    }
    if ((st = gmm_prepare(desc, ws, ws_bytes, pi, mu, cov, stream)) != GMM_OK) return st;
    hipLaunchKernelGGL(k_fit_reset, dim3(1), dim3(1), 0, stream, ctl, opts->max_iter,
                       opts->tol * (double)p.n);
    if (hipGetLastError() != hipSuccess) return GMM_E_HIP;

    // ---- one iteration, as launches on `stream`
    const int64_t n_pi = p.k, n_mu = p.k * p.d, n_cov = (int64_t)theta_cov_elems(p);
    const int commit_grid = (int)std::min<int64_t>(1024, (n_pi + n_mu + n_cov + 255) / 256);
    auto iteration = [&]() -> gmm_status {
        gmm_status s2 = gmm_em_step(desc, ws, ws_bytes, x, nullptr, stream);
        if (s2 != GMM_OK) return s2;
        if ((s2 = gmm_finalize(desc, ws, ws_bytes, nullptr, nullptr, nullptr, stream)) != GMM_OK) return s2;
        hipLaunchKernelGGL(k_fit_check, dim3(1), dim3(1), 0, stream, ctl, (const double*)(base + p.off_ll),
                           ll_hist);
        hipLaunchKernelGGL(k_fit_commit, dim3(commit_grid), dim3(256), 0, stream, (const FitCtl*)ctl,
                           (const float*)(base + p.off_pi), (const float*)(base + p.off_mu),
                           (const float*)(base + p.off_cov), n_pi, n_mu, n_cov, pi, mu, cov);
        return hipGetLastError() == hipSuccess ? GMM_OK : GMM_E_HIP;
    };

    // ---- capture it once (a non-null stream is needed), else launch directly
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    if (opts->use_graph && stream != nullptr) {
        if (hipStreamBeginCapture(stream, hipStreamCaptureModeThreadLocal) == hipSuccess) {
            const gmm_status sc = iteration();
            const hipError_t ec = hipStreamEndCapture(stream, &graph);
            if (sc != GMM_OK || ec != hipSuccess ||
                hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) != hipSuccess) {
                if (exec) hipGraphExecDestroy(exec);
                if (graph) hipGraphDestroy(graph);
                exec = nullptr;
                graph = nullptr;
                (void)hipGetLastError();
            }
        } else {
            (void)hipGetLastError();
        }
    }

    FitCtl h;
    memset(&h, 0, sizeof(h));
    int launched = 0;
    st = GMM_OK;
    while (launched < opts->max_iter) {
        const int b = std::min(opts->batch, opts->max_iter - launched);
        for (int i = 0; i < b && st == GMM_OK; ++i) {
            if (exec) st = hipGraphLaunch(exec, stream) == hipSuccess ? GMM_OK : GMM_E_HIP;
            else st = iteration();
        }
        launched += b;
        if (st != GMM_OK) break;
        if (hipStreamSynchronize(stream) != hipSuccess ||
            hipMemcpy(&h, ctl, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess) {
            st = GMM_E_HIP;
            break;
        }
        if (h.stop) break;
    }
    if (exec) hipGraphExecDestroy(exec);
    if (graph) hipGraphDestroy(graph);
    if (st != GMM_OK) return st;
    if (n_iter != nullptr) *n_iter = h.iter;
    // the workspace may hold iterations replayed after the stop: prepare it
    // for the committed parameters
    if ((st = gmm_prepare(desc, ws, ws_bytes, pi, mu, cov, stream)) != GMM_OK) return st;
    return hipStreamSynchronize(stream) == hipSuccess ? GMM_OK : GMM_E_HIP;
}

}  // extern "C"
