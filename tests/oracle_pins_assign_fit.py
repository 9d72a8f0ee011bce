"""Pins for the oracle's assignment, start and fit-loop functions
(oracle/gmm_assign_fit.py), each against something other than the oracle:

  * SplitMix64: the generator's first outputs from state 0 as published with
    its reference implementation (tests/golden/splitmix64_seed0.json);
  * Floyd's sampling: distinct, sorted, in range; every 2-subset of 5 items
    equally likely over many seeds (uniformity is what the algorithm proves);
  * the random-points start: its means are exactly the sampled rows;
  * top-m assignment: m = 1 is the argmax, m = K is scikit-learn's
    predict_proba sorted in decreasing order (responsibilities sum to 1),
    identical components are ordered by index, columns beyond K are empty;
  * the fit loop: scikit-learn's GaussianMixture run with the same start,
    tolerance and iteration cap (its convergence test is the same change of
    the per-point log-likelihood), and EM never lowers the log-likelihood.

Each pin takes the module `A` (gmm_assign_fit) and the core oracle `O`.
"""
from __future__ import annotations

import itertools
import json
import os
import warnings

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _problem(O, cov_type, n=500, d=3, k=4, seed=0, sep=5.0):
    rng = np.random.default_rng(seed)
    mu_t = sep * rng.standard_normal((k, d))
    z = rng.integers(0, k, size=n)
    x = mu_t[z] + rng.standard_normal((n, d))
    pi = rng.dirichlet(np.ones(k))
    mu = mu_t + 0.8 * rng.standard_normal((k, d))
    cov = {"diag": rng.uniform(0.5, 2.0, (k, d)), "iso": rng.uniform(0.5, 2.0, k),
           "full": np.stack([np.eye(d) * rng.uniform(0.5, 2.0) for _ in range(k)])}[cov_type]
    return x, O.Params(pi, mu, cov, cov_type)


def pin_splitmix64_reference(A, O):
    ref = json.load(open(os.path.join(GOLDEN, "splitmix64_seed0.json")))
    state = 0
    for want in ref["outputs_hex"]:
        state, out = A.splitmix64(state)
        assert out == int(want, 16), (hex(out), want)


def pin_floyd_sampling(A, O):
    for n, k, seed in ((10, 4, 1), (1000, 37, 99), (7, 7, 3), (5, 0, 2)):
        s = A.sample_distinct(n, k, seed)
        assert len(s) == k and len(set(s.tolist())) == k
        assert np.all(np.diff(s) > 0) and (k == 0 or (s[0] >= 0 and s[-1] < n))
    assert np.array_equal(A.sample_distinct(7, 7, 3), np.arange(7))
    counts = {}
    trials = 20000
    for seed in range(trials):
        counts[tuple(A.sample_distinct(5, 2, seed))] = counts.get(tuple(A.sample_distinct(5, 2, seed)), 0) + 1
    assert set(counts) == set(itertools.combinations(range(5), 2))
    freq = np.array(list(counts.values())) / trials
    assert np.all(np.abs(freq - 0.1) < 0.012), freq     # 5.6 sigma of a binomial(20000, 0.1)


def pin_random_points_start(A, O):
    x, _ = _problem(O, "diag", n=300, d=4)
    for ct in ("diag", "iso", "full"):
        p = A.init_random_points(x, 6, 12345, ct)
        idx = A.sample_distinct(300, 6, 12345)
        assert np.array_equal(p.mu, x[idx])
        assert np.array_equal(p.pi, np.full(6, 1.0 / 6))
        want = {"diag": np.ones((6, 4)), "iso": np.ones(6), "full": np.tile(np.eye(4), (6, 1, 1))}[ct]
        assert np.array_equal(p.cov, want)


def pin_topm(A, O):
    from sklearn.mixture import GaussianMixture
    sk_name = {"diag": "diag", "iso": "spherical", "full": "full"}
    for ct in ("diag", "iso", "full"):
        x, p = _problem(O, ct, seed=5)
        k = p.k
        _, _, arg = O.loglik(x, p, ridge_rel=0.0)
        idx1, g1, _ = A.assign_topm(x, p, 1, ridge_rel=0.0)
        assert np.array_equal(idx1[:, 0], arg)
        idx, gam, _ = A.assign_topm(x, p, k, ridge_rel=0.0)
        gm = GaussianMixture(n_components=k, covariance_type=sk_name[ct])
        gm.weights_, gm.means_, gm.covariances_ = p.pi, p.mu, p.cov
        prec = 1.0 / p.cov if ct != "full" else np.linalg.inv(p.cov)
        gm.precisions_cholesky_ = np.sqrt(prec) if ct != "full" else np.linalg.cholesky(prec)
        proba = gm.predict_proba(x)
        np.testing.assert_allclose(gam, -np.sort(-proba, axis=1), rtol=1e-9, atol=1e-15)
        np.testing.assert_allclose(np.take_along_axis(proba, idx, axis=1), gam, rtol=1e-9, atol=1e-15)
        np.testing.assert_allclose(gam.sum(axis=1), 1.0, rtol=1e-12)
        assert np.all(np.diff(gam, axis=1) <= 1e-15)
        # beyond K: empty columns
        idx9, gam9, _ = A.assign_topm(x[:10], p, k + 2, ridge_rel=0.0)
        assert np.all(idx9[:, k:] == -1) and np.all(gam9[:, k:] == 0.0)
    # a zero-weight component (log-joint -inf) is never listed
    x, p = _problem(O, "iso", k=3, seed=7)
    p.pi[1] = 0.0
    p.pi /= p.pi.sum()
    idx, gam, _ = A.assign_topm(x[:20], p, 3)
    assert np.all(idx[:, :2] != 1) and np.all(idx[:, 2] == -1) and np.all(gam[:, 2] == 0.0)
    # identical components: equal responsibilities, lower index first
    x, p = _problem(O, "diag", k=3, seed=6)
    p.mu[2], p.cov[2], p.pi[2] = p.mu[0], p.cov[0], p.pi[0]
    idx, gam, _ = A.assign_topm(x, p, 3)
    for i in range(x.shape[0]):
        r = idx[i].tolist()
        assert r.index(0) < r.index(2)
        j0, j2 = r.index(0), r.index(2)
        assert gam[i, j0] == gam[i, j2]


def pin_fit_sklearn(A, O):
    """The loop equals scikit-learn's GaussianMixture.fit from the same start
    (reg_covar 0, no variance floor): same number of iterations, the last
    per-point log-likelihood, and the final parameters."""
    from sklearn.exceptions import ConvergenceWarning
    from sklearn.mixture import GaussianMixture
    sk_name = {"diag": "diag", "iso": "spherical", "full": "full"}
    for ct, tol, cap in (("diag", 1e-4, 200), ("iso", 1e-3, 200), ("full", 1e-4, 200), ("diag", 0.0, 7)):
        x, p = _problem(O, ct, n=800, seed=8, sep=1.5)   # overlapping: slow convergence
        lls, pf, nit = A.fit_tol(x, p, tol, cap, var_floor=0.0, ridge_rel=0.0)
        prec = 1.0 / p.cov if ct != "full" else np.linalg.inv(p.cov)
        gm = GaussianMixture(n_components=p.k, covariance_type=sk_name[ct], reg_covar=0.0,
                             max_iter=cap, tol=tol, weights_init=p.pi, means_init=p.mu,
                             precisions_init=prec, random_state=0)
        with warnings.catch_warnings():
            warnings.simplefilter("ignore", ConvergenceWarning)
            gm.fit(x)
        assert nit == gm.n_iter_, (ct, nit, gm.n_iter_)
        np.testing.assert_allclose(lls[-1] / x.shape[0], gm.lower_bound_, rtol=1e-10)
        np.testing.assert_allclose(pf.pi, gm.weights_, rtol=1e-8)
        np.testing.assert_allclose(pf.mu, gm.means_, rtol=1e-8, atol=1e-10)
        np.testing.assert_allclose(pf.cov, gm.covariances_, rtol=1e-7, atol=1e-10)
        assert all(b >= a - 1e-9 * abs(a) for a, b in zip(lls, lls[1:]))
        if tol == 0.0:
            assert nit == cap


ALL_PINS = [pin_splitmix64_reference, pin_floyd_sampling, pin_random_points_start, pin_topm,
            pin_fit_sklearn]
