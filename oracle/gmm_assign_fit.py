"""Plain fp64 CPU oracle for the steps around the EM iteration: top-m soft
assignment, the seeded random-points start, and the EM loop with a
log-likelihood tolerance.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import or call this module; the product path
never does, and the two share no code.

Sources (web pages, cited by title and section):

* [Flash-GMM] "Flash-GMM: a memory-efficient kernel for scalable soft
  clustering" (ai-feeds.com/i/paper/2606.10896):
    - Key findings: soft responsibilities let a boundary vector belong to
      several clusters (the top responsibilities of a point);
    - Deployment: coarse quantiser of an IVF index with multi-cluster
      assignment;
    - Method, outputs: the fused step is called repeatedly until the
      log-likelihood converges.
* [LP-GMM] the low-precision GMM operator write-up (hotelren.com/news/5857197),
  section 1.1: training repeats E and M steps; inference needs the E-step.

Generators (published definitions, implemented here from them):
* SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable pseudorandom
  number generators", OOPSLA 2014), in its common 64-bit form: the state
  advances by the golden-ratio increment 0x9E3779B97F4A7C15 and each output
  is the state passed through the variant-13 mixer (xor-shift 30, multiply by
  0xBF58476D1CE4E5B9, xor-shift 27, multiply by 0x94D049BB133111EB,
  xor-shift 31).
* Floyd's algorithm for a uniform K-subset of {0..N-1} (J. Bentley, R. Floyd,
  "A sample of brilliance", CACM 1987): for j = N-K .. N-1 draw t uniform in
  [0, j]; take t, or j when t is already taken.

Readings of points the pages leave open: ties in the top-m order go to the lower
component index; the random draw in [0, j] is the generator's output modulo
j + 1; the start is K distinct points in increasing index order as means,
unit (co)variances and equal weights; the loop stops after iteration t >= 1
when |LL_t - LL_{t-1}| / N < tol, and returns the parameters that iteration's
M-step produced.
"""
from __future__ import annotations

import numpy as np

from .gmm_oracle import (DEFAULT_RIDGE_REL, DEFAULT_VAR_FLOOR, Params, em_step, log_joint,
                         log_normaliser, prepare)

MASK64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15


def splitmix64(state: int):
    """One SplitMix64 step: returns (new_state, 64-bit output)."""
    state = (state + GOLDEN) & MASK64
    z = state
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return state, z ^ (z >> 31)


def sample_distinct(n: int, k: int, seed: int) -> np.ndarray:
    """K distinct indices of {0..N-1} by Floyd's algorithm, sorted."""
    if not 0 <= k <= n:
        raise ValueError("need 0 <= k <= n")
    state = seed & MASK64
    chosen = set()
    for j in range(n - k, n):
        state, r = splitmix64(state)
        t = r % (j + 1)
        chosen.add(j if t in chosen else t)
    return np.array(sorted(chosen), dtype=np.int64)


def init_random_points(x: np.ndarray, k: int, seed: int, cov_type: str) -> Params:
    """EM start: K distinct data points (sample_distinct) as means, unit
    variances (identity for full covariance), weights 1/K."""
    x = np.asarray(x, dtype=np.float64)
    n, d = x.shape
    idx = sample_distinct(n, k, seed)
    cov = {"diag": np.ones((k, d)), "iso": np.ones(k), "full": np.tile(np.eye(d), (k, 1, 1))}[cov_type]
    return Params(np.full(k, 1.0 / k), x[idx].copy(), cov, cov_type)


def assign_topm(x: np.ndarray, p: Params, m: int, ridge_rel: float = DEFAULT_RIDGE_REL):
    """Per point the m components with the largest responsibilities, in
    decreasing order (ties: lower component index first), and those
    responsibilities gamma_nk = exp(a_nk - lse_n).  A component whose
    log-joint is -inf (zero weight) has responsibility exactly 0 and is not a
    member: it is never listed.  Columns past the listed components hold
    index -1 and responsibility 0.  Returns (idx [N, m], gamma [N, m], lse [N])."""
    x = np.asarray(x, dtype=np.float64)
    a = log_joint(x, p, prepare(p, ridge_rel))
    lse = log_normaliser(a)
    n, kk = a.shape
    idx = np.full((n, m), -1, dtype=np.int64)
    gam = np.zeros((n, m))
    ks = np.arange(kk)
    take = min(m, kk)
    for i in range(n):
        order = np.lexsort((ks, -a[i]))[:take]   # primary: larger a; then lower k
        order = order[np.isfinite(a[i, order])]
        idx[i, :order.size] = order
        gam[i, :order.size] = np.exp(a[i, order] - lse[i])
    return idx, gam, lse


def fit_tol(x: np.ndarray, p: Params, tol: float, max_iter: int,
            var_floor: float = DEFAULT_VAR_FLOOR, ridge_rel: float = DEFAULT_RIDGE_REL):
    """EM iterations from p until |LL_t - LL_{t-1}| / N < tol (t >= 1) or
    max_iter iterations.  Returns (LL per iteration, final parameters, number
    of iterations)."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0]
    lls = []
    for _ in range(max_iter):
        r = em_step(x, p, var_floor, ridge_rel)
        lls.append(r.ll)
        p = r.params
        if len(lls) >= 2 and abs(lls[-1] - lls[-2]) / n < tol:
            break
    return lls, p, len(lls)
