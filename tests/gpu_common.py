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


MIN_MASS = 1.0    # components lighter than one point's responsibility: absolute bound below
LIGHT_FRAC = 0.05


def check_step(ref, ll, st, theta, tol=FP32_TOL, what="", xd=None):
    """One-step parity: LL(theta_t), statistics and theta_{t+1}.

    The statistics s0 / s1 / s2 and pi are gated over all components, mu' and
    the variances of components holding at least MIN_MASS points at `tol`.
    A lighter component's mu' = s1/s0 is a ratio of tail responsibilities:
    its points sit far out, where the fp32 score error (about 2^-21 of |S|)
    moves each responsibility by up to a few per cent, and the ratio moves by
    that fraction of the spread of those points.  Its mean is therefore held
    to within LIGHT_FRAC of the data's range in each dimension, and its
    variance to within LIGHT_FRAC of the squared range (xd: the stored X)."""
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
    print(what, " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    if not heavy.all():
        assert xd is not None, (what, "light components need the data range for their bound")
        rng = np.ptp(np.asarray(xd, np.float64), axis=0)
        light = ~heavy
        dmu = np.abs(mu_g[light] - ref.params.mu[light]) / (LIGHT_FRAC * rng)
        dcv = np.abs(cov_g[light] - ref.params.cov[light]) / (LIGHT_FRAC * rng * rng)
        print(f"   light components {np.nonzero(light)[0].tolist()} (s0 < {MIN_MASS}): "
              f"|d mu'| / ({LIGHT_FRAC} range) max {dmu.max():.2e}, "
              f"|d var'| / ({LIGHT_FRAC} range^2) max {dcv.max():.2e}", flush=True)
        errs["light_mu"], errs["light_cov"] = float(dmu.max()), float(dcv.max())
        assert errs["light_mu"] <= 1.0 and errs["light_cov"] <= 1.0, (what, errs)
    bad = {k: v for k, v in errs.items() if k not in ("light_mu", "light_cov") and not v <= tol}
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


# ---- reduced-precision (fp16 operand) paths ---------------------------------

LOG2E = 1.4426950408889634
FP16_U = 2.0 ** -11


def fp16_score_error_nats(theta, x, cov_type):
    """Estimated rounding error, in nats, of each component's fp16
    expanded-form score [x^2 | x] . panel near its own mean, from theta and X
    alone (numpy, no library output): two fp16 roundings of relative size
    2^-11 on each term A y^2 and B y with y = x - c measured from the data
    mean c, at a point |mu - c| + 3 sigma out, random signs.  A component whose
    variance collapsed (say onto one point at the variance floor) gives
    thousands of nats: the expanded form cannot resolve it in fp16."""
    pi, mu, cov = (np.asarray(t, np.float64) for t in theta)
    c = np.asarray(x, np.float64).mean(axis=0)
    var = cov[:, None] * np.ones_like(mu) if cov_type == "iso" else cov
    mc = mu - c
    yt = np.abs(mc) + 3.0 * np.sqrt(np.abs(var))
    ta = 0.5 * LOG2E * yt * yt / var
    tb = LOG2E * mc * yt / var
    bits = np.sqrt(np.sum(ta * ta + tb * tb, axis=1)) * FP16_U * np.sqrt(2.0 / 3.0)
    return bits * np.log(2.0)


ILL_COND_NATS = 4.0


def ill_conditioned(theta, x, cov_type):
    """Indices of components whose fp16 expanded-form score is estimated to
    be off by more than ILL_COND_NATS near their own mean (fp16_score_error_nats)."""
    return np.nonzero(fp16_score_error_nats(theta, x, cov_type) > ILL_COND_NATS)[0].tolist()


def point_score_error_nats(theta, x, cov_type):
    """The error model of fp16_score_error_nats at every (point, component):
    the terms A y_d^2 and B y_d of the point's own y = x - c, two fp16
    roundings each with random signs.  Returns an [N, K] array in nats."""
    pi, mu, cov = (np.asarray(t, np.float64) for t in theta)
    x = np.asarray(x, np.float64)
    c = x.mean(axis=0)
    y2 = (x - c) ** 2
    var = cov[:, None] * np.ones_like(mu) if cov_type == "iso" else cov
    a = 0.5 * LOG2E / var
    b = LOG2E * (mu - c) / var
    s = (y2 * y2) @ (a * a).T + y2 @ (b * b).T
    return np.sqrt(np.maximum(s, 0.0)) * FP16_U * np.sqrt(2.0 / 3.0) * np.log(2.0)


def gamma_error_bound(x, p, theta32, cov_type, margin=3.0, exact_nats=2.0):
    """Bound on |gamma_gpu - gamma| per (point, component) from the fp16
    score errors: E_nk = margin x point_score_error_nats (a component whose
    fp16_score_error_nats exceeds exact_nats is taken as scored exactly in
    fp32, E = 1e-4).  With every score of point n off by at most E_nj,
    gamma'_nk = gamma_nk e^d_k / sum_j gamma_nj e^d_j lies between
    gamma e^-E_k / (gamma e^-E_k + sum_{j != k} gamma_nj e^E_j) and
    gamma e^E_k / (gamma e^E_k + sum_{j != k} gamma_nj e^-E_j): the bound is
    the larger distance of the two from gamma_nk.  gamma from the oracle.
    Returns (bound, gamma)."""
    exact = fp16_score_error_nats(theta32, x, cov_type) > exact_nats
    e = np.minimum(margin * point_score_error_nats(theta32, x, cov_type), 60.0)   # e^60: still finite
    e[:, exact] = 1e-4
    a = oracle.log_joint(x, p, oracle.prepare(p))
    lse = np.logaddexp.reduce(a, axis=1)
    g = np.exp(a - lse[:, None])
    gu = g * np.exp(e)
    gd = g * np.exp(-e)
    rest_up = gu.sum(axis=1, keepdims=True) - gu   # sum_{j != k} gamma_nj e^E_nj
    rest_dn = gd.sum(axis=1, keepdims=True) - gd
    with np.errstate(invalid="ignore", divide="ignore"):
        hi = np.where(gu > 0, gu / (gu + rest_dn), 0.0)
        lo = np.where(gd > 0, gd / (gd + rest_up), 0.0)
    return np.maximum(hi - g, g - lo), g


def check_params_bounded(ref, st, theta, x, B, g, cov_type, stat_u=FP16_U, what=""):
    """s0, mu and the variances of every component against the oracle's,
    element by element, within the error that the responsibility bound B
    (gamma_error_bound) propagates: s0 by sum_n B_nk, and to first order mu
    by sum_n B_nk |x_n - mu_k| / s0_k, the variance by sum_n B_nk |(x_n -
    mu_k)^2 - var_k| / s0_k (isotropic: the mean over dimensions).  Plus the
    rounding of the statistics operands, relative stat_u each, worst case:
    y = x - c (c the data centre) staged in fp16 moves mu by
    stat_u sum_n gamma_nk |y_n| / s0_k and, through the mean subtracted in
    the variance, the variance by 2 |mu_k - c| times that; y^2 staged in
    fp16 moves the variance by stat_u sum_n gamma_nk y_n^2 / s0_k.  And a
    floor for the fp32 arithmetic (1e-3 relative, 1e-4 of the largest).
    The first-order propagation to mu and the variance holds while the mass
    bound is small against the mass: components with sum_n B_nk > s0_k / 4
    (their weight is not determined at this precision) have s0 checked and
    their mean and variance reported, not compared."""
    x = np.asarray(x, np.float64)
    n, d = x.shape
    c = x.mean(axis=0)
    s0 = np.asarray(ref.nk, np.float64)
    mu, var = ref.params.mu, ref.params.cov
    bs0 = B.sum(axis=0)
    bmu = np.zeros_like(mu)
    bvar = np.zeros_like(var)
    for k in np.nonzero((bs0 > 0) | (s0 > 0))[0]:
        live = (B[:, k] > 0) | (g[:, k] > 0)
        dx = x[live] - mu[k]
        yc = np.abs(x[live] - c)
        w = B[live, k] / max(s0[k], 1e-300)
        wg = stat_u * g[live, k] / max(s0[k], 1e-300)
        rmu = wg @ yc                             # per dimension
        bmu[k] = w @ np.abs(dx) + rmu
        mc = np.abs(mu[k] - c)
        if cov_type == "iso":
            bvar[k] = (w @ np.abs((dx * dx).mean(axis=1) - var[k]) + wg @ (yc * yc).mean(axis=1) +
                       np.mean(2.0 * mc * rmu))
        else:
            bvar[k] = w @ np.abs(dx * dx - var[k]) + wg @ (yc * yc) + 2.0 * mc * rmu
    heavy = s0 >= 1e-3 * n / max(len(s0), 1)   # empty components keep theta: not compared
    loose = heavy & (bs0 > 0.25 * s0)
    if loose.any():
        print(f"   {what}: {int(loose.sum())} components with mass bound above s0 / 4 "
              f"(first {np.nonzero(loose)[0][:8].tolist()}): mean and variance not compared", flush=True)
    heavy &= ~loose
    out = {}
    for name, got, want, bnd in (("s0", st.s0.cpu().numpy(), s0, bs0),
                                 ("mu", theta[1].cpu().numpy(), mu, bmu),
                                 ("var", theta[2].cpu().numpy(), var, bvar)):
        got = np.asarray(got, np.float64).reshape(np.shape(want))
        err = np.abs(got - want)
        allow = bnd + 1e-3 * np.abs(want) + 1e-4 * np.max(np.abs(want))
        ratio = err / allow
        if name != "s0":
            ratio[~heavy] = 0.0
        worst = float(np.max(ratio)) if ratio.size else 0.0
        i = np.unravel_index(int(np.argmax(ratio)), ratio.shape) if ratio.size else ()
        out[name] = worst
        print(f"   {what} {name}: worst err/bound {worst:.3f} at {i} (err {err[i] if ratio.size else 0:.3e}, "
              f"bound {allow[i] if ratio.size else 0:.3e})", flush=True)
    bad = {k: v for k, v in out.items() if not v <= 1.0}
    assert not bad, (what, bad)
    return out


def oracle_stats_chunked(x, p, chunk=8192, workers=8, **kw):
    """The oracle's em_step over consecutive chunks of points in a thread
    pool; returns (LL, s0, s1, s2) summed over the chunks in chunk order (the
    E-step statistics of the whole set: each chunk's sums are exact fp64
    sums over its points)."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    parts = [x[lo:lo + chunk] for lo in range(0, x.shape[0], chunk)]
    with threadpool_limits(limits=1), ThreadPoolExecutor(workers) as ex:
        res = list(ex.map(lambda a: oracle.em_step(a, p, **kw), parts))
    ll = sum(r.ll for r in res)
    s0 = sum(r.nk for r in res)
    s1 = sum(r.s1 for r in res)
    s2 = sum(r.s2 for r in res)
    return ll, s0, s1, s2


def stats_elementwise(got, ref, rtol, atol_frac, what=""):
    """Element-by-element check |got - ref| <= rtol |ref| + atol_frac max|ref|;
    returns the largest ratio of the error to that allowance."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    allow = rtol * np.abs(ref) + atol_frac * np.max(np.abs(ref))
    err = np.abs(got - ref)
    worst = float(np.max(err / allow)) if err.size else 0.0
    i = int(np.argmax(err / allow)) if err.size else 0
    print(f"   {what}: worst err/allowance {worst:.3f} at flat index {i} "
          f"(got {got.ravel()[i]:.6e}, ref {ref.ravel()[i]:.6e})", flush=True)
    assert worst <= 1.0, (what, worst)
    return worst
