"""Helpers shared by the GPU parity tests: running the HIP path through the
binding and the oracle on the same inputs."""
import numpy as np
import torch

import oracle
from soft_clustering_amd import synth
from tests import metrics

FP32_TOL = 1e-4   # fp32 path: LL and parameters, relative


def to_dev(*arrs):
    return [torch.as_tensor(np.ascontiguousarray(a), dtype=torch.float32).cuda() for a in arrs]


def params64(cov_type, pi, mu, cov):
    f = lambda t: t.detach().double().cpu().numpy() if torch.is_tensor(t) else np.asarray(t, np.float64)
    return oracle.Params(f(pi), f(mu), f(cov), cov_type)


def gpu_step(gm, x, pi, mu, cov, prepare=True):
    """One EM iteration on the GPU; returns (ll, stats, (pi', mu', cov'))."""
    if prepare:
        gm.prepare(pi, mu, cov)
    ll = torch.zeros(1, dtype=torch.float64, device="cuda")
    gm.em_step(x, ll)
    po = torch.empty_like(pi)
    mo = torch.empty_like(mu)
    co = torch.empty_like(cov)
    gm.finalize(po, mo, co)
    st = gm.get_stats()          # reduced by finalize
    torch.cuda.synchronize()
    return float(ll.item()), st, (po, mo, co)


MIN_MASS = 1.0    # components lighter than one point's responsibility: reported, not gated


def check_step(ref, ll, st, theta, tol=FP32_TOL, what=""):
    """One-step parity: LL(theta_t), statistics and theta_{t+1}.

    The statistics s0 / s1 / s2 are gated over all components.  The new mean
    and covariance of a component holding less than MIN_MASS points of
    responsibility are the ratio of tail responsibilities that fp32 scores
    resolve only to about 1e-4..1e-3, so those parameters are reported, not
    gated (their absolute error is already bounded by the statistics)."""
    heavy = np.asarray(ref.nk) >= MIN_MASS
    mu_g, cov_g = theta[1].cpu().numpy(), theta[2].cpu().numpy()
    errs = {
        "ll": metrics.rel(ll, ref.ll),
        "s0": metrics.rel_inf(st.s0.cpu().numpy(), ref.nk),
        "s1": metrics.rel_inf(st.s1.cpu().numpy(), ref.s1),
        "s2": metrics.rel_inf(st.s2.cpu().numpy(), ref.s2),
        "pi": metrics.rel_inf(theta[0].cpu().numpy(), ref.params.pi),
        "mu": metrics.rel_inf(mu_g[heavy], ref.params.mu[heavy]) if heavy.any() else 0.0,
        "cov": metrics.rel_inf(cov_g[heavy], ref.params.cov[heavy]) if heavy.any() else 0.0,
    }
    if not heavy.all():
        print(f"   light components {np.nonzero(~heavy)[0].tolist()}: mu rel "
              f"{metrics.rel_inf(mu_g[~heavy], ref.params.mu[~heavy]):.2e} (not gated)", flush=True)
    print(what, " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, (what, bad)
    return errs


def workload_inputs(name, n=None, device="cpu"):
    w = synth.WORKLOADS[name]
    if n is not None:
        w = w.with_n(n, f"-n{n}")
    mix = synth.make_mixture(w)
    x = synth.sample_points(w, mix, device=device)
    pi, mu, cov = synth.init_params(w, x)
    return w, x, (pi, mu, cov)
