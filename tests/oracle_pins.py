"""Pins that tie the fp64 oracle to something other than itself.

Each pin takes the oracle module `O` as an argument and raises AssertionError
when the oracle disagrees with:
  * a third-party library routine (scipy's multivariate normal log-density,
    scikit-learn's GaussianMixture EM iteration, scipy's logsumexp);
  * a closed form (one component: sample mean / population variance and the
    log-likelihood at the MLE; the two-component posterior is a logistic);
  * brute-force enumeration of every hard assignment on tiny inputs;
  * an invariant (rows of responsibilities sum to 1, EM never lowers the
    log-likelihood, translation / scale / permutation equivariance, chunking
    does not change the answer);
  * an independent eigen-decomposition route for the full covariance.

tests/test_oracle_pins.py runs them on the real oracle and
tests/test_oracle_mutations.py runs them on deliberately broken copies of the
oracle (the checker's self-test from the operator-debugging article, section
7.2), which must each fail at least one pin.
"""
from __future__ import annotations

import itertools
import math
import warnings

import numpy as np
from scipy import stats
from scipy.special import logsumexp

RTOL = 1e-10


def _close(a, b, rtol=RTOL, atol=0.0, what=""):
    np.testing.assert_allclose(a, b, rtol=rtol, atol=atol, err_msg=what)


def _random_problem(O, cov_type, n=400, d=4, k=3, seed=0, sep=4.0):
    """Points from a random mixture plus a different random parameter set."""
    rng = np.random.default_rng(seed)
    mu_true = sep * rng.standard_normal((k, d))
    z = rng.integers(0, k, size=n)
    x = mu_true[z] + rng.standard_normal((n, d)) * rng.uniform(0.5, 1.5, size=(k, d))[z]
    pi = rng.dirichlet(np.ones(k))
    mu = mu_true + 0.7 * rng.standard_normal((k, d))
    if cov_type == "diag":
        cov = rng.uniform(0.5, 2.0, size=(k, d))
    elif cov_type == "iso":
        cov = rng.uniform(0.5, 2.0, size=k)
    else:
        cov = np.empty((k, d, d))
        for j in range(k):
            a = rng.standard_normal((d, d))
            cov[j] = a @ a.T / d + 0.5 * np.eye(d)
    return x, O.Params(pi, mu, cov, cov_type)


def _dense_cov(p, k):
    d = p.mu.shape[1]
    if p.cov_type == "diag":
        return np.diag(p.cov[k])
    if p.cov_type == "iso":
        return p.cov[k] * np.eye(d)
    return p.cov[k]


def _scipy_log_joint(p, x):
    return np.stack([math.log(p.pi[k]) + stats.multivariate_normal(p.mu[k], _dense_cov(p, k)).logpdf(x)
                     for k in range(p.mu.shape[0])], axis=1).reshape(x.shape[0], -1)


# ---------------------------------------------------------------------------

def pin_rows_sum_to_one(O):
    for ct in ("diag", "iso", "full"):
        x, p = _random_problem(O, ct, seed=1)
        prep = O.prepare(p, 0.0)
        a = O.log_joint(x, p, prep)
        g = O.responsibilities(a, O.log_normaliser(a))
        _close(g.sum(axis=1), np.ones(x.shape[0]), rtol=1e-14, what=ct)
        assert np.all(g >= 0.0)


def pin_k1_closed_form(O):
    """One component: gamma == 1, mu' = sample mean, var' = population variance,
    pi' = 1; at the MLE, LL = -(N/2) (D (1 + log 2 pi) + log |C_hat|)."""
    rng = np.random.default_rng(2)
    n, d = 300, 5
    x = 3.0 + rng.standard_normal((n, d)) * np.array([0.5, 1.0, 2.0, 0.8, 1.3])
    mean = x.mean(axis=0)
    for ct in ("diag", "iso", "full"):
        if ct == "diag":
            cov0, hat = np.ones((1, d)), x.var(axis=0)[None, :]
            logdet = np.sum(np.log(hat))
        elif ct == "iso":
            cov0, hat = np.ones(1), np.array([x.var(axis=0).mean()])
            logdet = d * np.log(hat[0])
        else:
            cov0, hat = np.eye(d)[None], np.cov(x.T, bias=True)[None]
            logdet = np.linalg.slogdet(hat[0])[1]
        p0 = O.Params(np.ones(1), np.zeros((1, d)), cov0, ct)
        r = O.em_step(x, p0, var_floor=0.0, ridge_rel=0.0)
        _close(r.nk, [n], rtol=1e-15, what=ct)
        _close(r.params.pi, [1.0], rtol=1e-15)
        _close(r.params.mu[0], mean, rtol=1e-12, what=ct)
        _close(r.params.cov, hat, rtol=1e-11, what=ct)
        r2 = O.em_step(x, r.params, var_floor=0.0, ridge_rel=0.0)
        ll_mle = -0.5 * n * (d * (1.0 + math.log(2.0 * math.pi)) + logdet)
        _close(r2.ll, ll_mle, rtol=1e-12, what=ct)


def pin_logpdf_scipy(O):
    for ct in ("diag", "iso", "full"):
        x, p = _random_problem(O, ct, seed=3, d=6, k=4)
        a = O.log_joint(x, p, O.prepare(p, 0.0))
        _close(a, _scipy_log_joint(p, x), rtol=1e-11, what=ct)
        ll, lse, arg = O.loglik(x, p, ridge_rel=0.0)
        _close(lse, logsumexp(_scipy_log_joint(p, x), axis=1), rtol=1e-11)
        assert np.array_equal(arg, np.argmax(_scipy_log_joint(p, x), axis=1))


def pin_sklearn(O):
    """One EM iteration equals scikit-learn's (reg_covar = 0, given init)."""
    from sklearn.exceptions import ConvergenceWarning
    from sklearn.mixture import GaussianMixture
    sk_name = {"diag": "diag", "iso": "spherical", "full": "full"}
    for ct in ("diag", "iso", "full"):
        x, p = _random_problem(O, ct, seed=4, n=600, d=5, k=4)
        if ct == "full":
            prec = np.linalg.inv(p.cov)
        else:
            prec = 1.0 / p.cov
        gm = GaussianMixture(n_components=p.k, covariance_type=sk_name[ct], reg_covar=0.0,
                             max_iter=1, tol=0.0, weights_init=p.pi, means_init=p.mu,
                             precisions_init=prec, random_state=0)
        with warnings.catch_warnings():
            warnings.simplefilter("ignore", ConvergenceWarning)
            gm.fit(x)
        r = O.em_step(x, p, var_floor=0.0, ridge_rel=0.0)
        _close(r.ll / x.shape[0], gm.lower_bound_, rtol=1e-12, what=ct)
        _close(r.params.pi, gm.weights_, rtol=1e-11, what=ct)
        _close(r.params.mu, gm.means_, rtol=1e-11, atol=1e-12, what=ct)
        _close(r.params.cov, gm.covariances_, rtol=1e-10, what=ct)


def pin_bruteforce(O):
    """Enumerate all K^N hard assignments z: log p(X) = logsumexp_z log p(X, z),
    gamma_nk = P(z_n = k | X), expected statistics by enumeration."""
    rng = np.random.default_rng(5)
    n, d, k = 6, 2, 3
    for ct in ("diag", "iso", "full"):
        x, p = _random_problem(O, ct, n=n, d=d, k=k, seed=6, sep=1.5)
        table = _scipy_log_joint(p, x)               # log pi_k + log N(x_n | k)
        zs = np.array(list(itertools.product(range(k), repeat=n)))
        logp = table[np.arange(n)[None, :], zs].sum(axis=1)
        log_px = logsumexp(logp)
        post = np.exp(logp - log_px)                  # P(z | X)
        onehot = (zs[:, :, None] == np.arange(k)[None, None, :]).astype(float)
        gamma = np.einsum("z,znk->nk", post, onehot)
        nk = gamma.sum(axis=0)
        mu_new = gamma.T @ x / nk[:, None]
        r = O.em_step(x, p, var_floor=0.0, ridge_rel=0.0)
        _close(r.ll, log_px, rtol=1e-12, what=ct)
        _close(r.nk, nk, rtol=1e-11, what=ct)
        _close(r.params.mu, mu_new, rtol=1e-10, atol=1e-12, what=ct)
        # expected centred second moments under P(z | X)
        if ct == "diag":
            var = np.stack([gamma[:, j] @ (x - mu_new[j]) ** 2 for j in range(k)]) / nk[:, None]
        elif ct == "iso":
            var = np.array([gamma[:, j] @ np.sum((x - mu_new[j]) ** 2, axis=1) for j in range(k)]) / (d * nk)
        else:
            var = np.stack([((x - mu_new[j]) * gamma[:, j:j + 1]).T @ (x - mu_new[j]) for j in range(k)]) / nk[:, None, None]
        _close(r.params.cov, var, rtol=1e-10, what=ct)
    # well separated: mu' is the per-cluster sample mean
    centers = np.array([[0.0, 0.0], [40.0, 0.0], [0.0, 40.0]])
    z = np.array([0, 0, 1, 1, 2, 2, 2])
    x = centers[z] + rng.standard_normal((7, 2))
    p = O.Params(np.full(3, 1 / 3), centers, np.ones((3, 2)), "diag")
    r = O.em_step(x, p, var_floor=0.0)
    _close(r.params.mu, np.stack([x[z == j].mean(axis=0) for j in range(3)]), rtol=1e-12)


def pin_monotone(O):
    for ct in ("diag", "iso", "full"):
        x, p = _random_problem(O, ct, seed=7, n=500, d=3, k=4, sep=2.5)
        lls, _ = O.fit(x, p, 15, var_floor=0.0, ridge_rel=0.0)
        assert all(b >= a - 1e-12 * abs(a) for a, b in zip(lls, lls[1:])), (ct, lls)


def pin_identical_components(O):
    rng = np.random.default_rng(8)
    x = rng.standard_normal((50, 3))
    pi = np.array([0.1, 0.2, 0.3, 0.4])
    p = O.Params(pi, np.tile([0.5, -1.0, 2.0], (4, 1)), np.tile([1.0, 2.0, 0.5], (4, 1)), "diag")
    a = O.log_joint(x, p, O.prepare(p))
    g = O.responsibilities(a, O.log_normaliser(a))
    _close(g, np.tile(pi, (50, 1)), rtol=1e-14)


def pin_logistic(O):
    x, p = _random_problem(O, "diag", seed=9, k=2, sep=1.0)
    t = _scipy_log_joint(p, x)
    a = O.log_joint(x, p, O.prepare(p))
    g = O.responsibilities(a, O.log_normaliser(a))
    _close(g[:, 0], 1.0 / (1.0 + np.exp(t[:, 1] - t[:, 0])), rtol=1e-11)


def pin_far_outlier(O):
    """A point far from every component: every exp would underflow without the
    max shift (the 'underflow black hole' of the low-precision write-up,
    section 4.2); with it gamma stays finite and one-hot."""
    x, p = _random_problem(O, "diag", seed=10)
    x = np.vstack([x, np.full((1, x.shape[1]), 1e3)])
    a = O.log_joint(x, p, O.prepare(p))
    lse = O.log_normaliser(a)
    g = O.responsibilities(a, lse)
    assert np.all(np.isfinite(lse)) and np.all(np.isfinite(g))
    _close(g[-1].max(), 1.0, rtol=1e-12)
    _close(lse[-1], logsumexp(a[-1]), rtol=1e-14)


def pin_equivariance(O):
    for ct in ("diag", "iso", "full"):
        x, p = _random_problem(O, ct, seed=11)
        r = O.em_step(x, p)
        c = np.array([3.0, -7.0, 0.5, 11.0])
        rt = O.em_step(x + c, O.Params(p.pi, p.mu + c, p.cov, ct))
        _close(rt.ll, r.ll, rtol=1e-11, what=ct)
        _close(rt.params.mu, r.params.mu + c, rtol=1e-11, atol=1e-11)
        _close(rt.params.cov, r.params.cov, rtol=1e-9, atol=1e-12)
        s = 2.5
        rs = O.em_step(s * x, O.Params(p.pi, s * p.mu, s * s * p.cov, ct))
        _close(rs.ll, r.ll - x.shape[0] * x.shape[1] * math.log(s), rtol=1e-11, what=ct)
        _close(rs.params.mu, s * r.params.mu, rtol=1e-11, atol=1e-12)
        _close(rs.params.cov, s * s * r.params.cov, rtol=1e-10)
        perm = np.array([2, 0, 1])
        rp = O.em_step(x[::-1], O.Params(p.pi[perm], p.mu[perm], p.cov[perm], ct))
        _close(rp.ll, r.ll, rtol=1e-12)
        _close(rp.params.pi, r.params.pi[perm], rtol=1e-11)
        _close(rp.params.mu, r.params.mu[perm], rtol=1e-11, atol=1e-12)
        _close(rp.params.cov, r.params.cov[perm], rtol=1e-10, atol=1e-13)


def pin_full_eigen_route(O, d=8, k=3):
    """C = Q diag(lam) Q^T: log|C + eps I| = sum log(lam + eps) and
    d2 = |(lam + eps)^{-1/2} Q^T (x - mu)|^2, a route without Cholesky."""
    rng = np.random.default_rng(12)
    qs, lams, covs = [], [], []
    for _ in range(k):
        q, rr = np.linalg.qr(rng.standard_normal((d, d)))
        q = q * np.sign(np.diag(rr))
        lam = 10.0 ** rng.uniform(-1.5, 1.5, size=d)
        qs.append(q), lams.append(lam), covs.append(q @ np.diag(lam) @ q.T)
    mu = 5.0 * rng.standard_normal((k, d))
    x = 5.0 * rng.standard_normal((200, d))
    p = O.Params(np.full(k, 1.0 / k), mu, np.stack(covs), "full")
    ridge_rel = 1e-3
    prep = O.prepare(p, ridge_rel)
    d2 = O.sq_mahalanobis(x, p, prep)
    for j in range(k):
        eps = ridge_rel * np.sum(lams[j]) / d
        _close(prep.ridge[j], eps, rtol=1e-12)
        _close(prep.logdet[j], np.sum(np.log(lams[j] + eps)), rtol=1e-10, atol=1e-12)
        w = (x - mu[j]) @ qs[j] / np.sqrt(lams[j] + eps)
        _close(d2[:, j], np.sum(w * w, axis=1), rtol=1e-9)


def pin_ridge_rule(O):
    """eps = ridge_rel * trace / D always; a failing pivot escalates eps x10."""
    cov = np.diag([1.0, 1.0, -0.01])
    L, eps, retries = O.ridged_cholesky(cov, 1e-3)
    tr = np.trace(cov) / 3
    assert retries == 2, retries
    _close(eps, 1e-3 * tr * 100, rtol=1e-12)
    _close(L @ L.T, cov + eps * np.eye(3), rtol=1e-12, atol=1e-15)
    try:
        O.ridged_cholesky(np.diag([1.0, 1.0, -50.0]), 1e-3)
    except O.NotPositiveDefinite:
        pass
    else:
        raise AssertionError("an indefinite covariance must be reported")
    a = np.array([[4.0, 2.0, 0.4], [2.0, 5.0, 1.0], [0.4, 1.0, 3.0]])
    L = O.cholesky_lower(a)
    _close(L, np.linalg.cholesky(a), rtol=1e-14)


def pin_floor_and_empty(O):
    rng = np.random.default_rng(13)
    x = rng.standard_normal((100, 3))
    x[:, 1] = 0.25                                 # a dimension with zero variance
    mu = np.array([[0.0, 0.25, 0.0], [1e4, 1e4, 1e4]])   # component 1 is empty
    p = O.Params(np.array([0.5, 0.5]), mu, np.array([[1.0, 1.0, 1.0], [2.0, 3.0, 4.0]]), "diag")
    r = O.em_step(x, p, var_floor=1e-6)
    assert r.params.cov[0, 1] == 1e-6
    assert r.nk[1] < O.EMPTY_NK
    assert np.array_equal(r.params.mu[1], mu[1]) and np.array_equal(r.params.cov[1], p.cov[1])
    _close(r.params.pi, r.nk / 100.0, rtol=1e-15)
    r2 = O.em_step(x, r.params)
    assert np.isfinite(r2.ll)


def pin_chunk_invariance(O):
    for ct in ("diag", "full"):
        x, p = _random_problem(O, ct, seed=14, n=333)
        a = O.em_step(x, p, chunk=1 << 16)
        b = O.em_step(x, p, chunk=7)
        _close(b.ll, a.ll, rtol=1e-13)
        _close(b.params.mu, a.params.mu, rtol=1e-12, atol=1e-14)
        _close(b.params.cov, a.params.cov, rtol=1e-12, atol=1e-14)


ALL_PINS = [
    pin_rows_sum_to_one, pin_k1_closed_form, pin_logpdf_scipy, pin_sklearn, pin_bruteforce,
    pin_monotone, pin_identical_components, pin_logistic, pin_far_outlier, pin_equivariance,
    pin_full_eigen_route, pin_ridge_rule, pin_floor_and_empty, pin_chunk_invariance,
]
