"""Plain fp64 CPU oracle for one Gaussian-mixture EM iteration.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import or call this module; the product path
(the HIP library and its Python binding) never does, and the two share no code.

Sources (web pages, cited by title and section):

* [LP-GMM]   the write-up on building a low-precision GMM operator
             (hotelren.com/news/5857197), sections 1.1-1.3, 3.1-3.2, 4.1-4.2.
* [Flash-GMM] "Flash-GMM: a memory-efficient kernel for scalable soft
             clustering" (ai-feeds.com/i/paper/2606.10896), section "Method"
             (inputs and modelling assumptions; fused E-M step; outputs).
* [ops-debug] the operator-debugging toolkit article (2kiu.com/news/5842513),
             section 3.1 (naive-loop and fp64 references).

What it computes is the textbook EM iteration, slowly and directly:

  * every point/component log-joint a_nk = log pi_k + log N(x_n | mu_k, C_k),
    with the Gaussian density in its centred form (no expansion of the
    quadratic, so no cancellation);
  * the per-point normaliser lse_n = log sum_k exp(a_nk) by the max-shift
    rule, and the responsibilities G_nk = exp(a_nk - lse_n), MATERIALISED
    per chunk of points (the oracle is allowed the N x K matrix the GPU path
    never writes);
  * the M-step: N_k = sum_n G_nk, mu'_k = sum_n G_nk x_n / N_k, and the new
    covariance centred about mu'_k in a second pass; pi'_k = N_k / N.

Precision: every operation is IEEE fp64 (numpy float64).  X is whatever the
caller stored (fp32 / fp16 / bf16 values), upcast exactly to fp64.

Readings of points the pages leave open:
  * LL is the total sum_n lse_n under the parameters the E-step used.
  * Variances are the maximum-likelihood ones (divide by N_k), clamped below
    at var_floor (a clamp keeps EM monotone; an additive floor would not).
  * Full covariance: a ridge eps = ridge_rel * |trace(C)|/D is always added
    before the Cholesky factorisation; a failing pivot multiplies eps by 10
    (at least to 1e-3 |trace(C)|/D), up to three times, and is flagged.
  * A component with N_k < EMPTY_NK keeps its mean and covariance; its weight
    becomes N_k / N.

Parity pins for every function live in tests/test_oracle_pins.py; none is
"parity unpinned".
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

LOG_2PI = math.log(2.0 * math.pi)
EMPTY_NK = 1e-6          # a component with fewer "points" than this is empty
DEFAULT_VAR_FLOOR = 1e-6
DEFAULT_RIDGE_REL = 1e-3  # [LP-GMM] 4.1: eps = 1e-3 * trace(Sigma) / D
RIDGE_RETRIES = 3
CHUNK = 1 << 16

COV_TYPES = ("diag", "iso", "full")


class NotPositiveDefinite(ValueError):
    """Raised when a covariance stays indefinite after every ridge retry."""


@dataclass
class Params:
    """GMM parameters theta = (pi, mu, cov) in fp64.

    pi  : [K]        mixing weights
    mu  : [K, D]     means
    cov : [K, D]     per-dimension variances   (cov_type "diag")
          [K]        one variance per component (cov_type "iso")
          [K, D, D]  covariance matrices        (cov_type "full")
    """
    pi: np.ndarray
    mu: np.ndarray
    cov: np.ndarray
    cov_type: str

    def __post_init__(self):
        if self.cov_type not in COV_TYPES:
            raise ValueError(f"cov_type must be one of {COV_TYPES}")
        self.pi = np.asarray(self.pi, dtype=np.float64)
        self.mu = np.asarray(self.mu, dtype=np.float64)
        self.cov = np.asarray(self.cov, dtype=np.float64)
        K, D = self.mu.shape
        want = {"diag": (K, D), "iso": (K,), "full": (K, D, D)}[self.cov_type]
        if self.pi.shape != (K,) or self.cov.shape != want:
            raise ValueError("inconsistent parameter shapes")

    @property
    def k(self) -> int:
        return self.mu.shape[0]

    @property
    def d(self) -> int:
        return self.mu.shape[1]


@dataclass
class Prepared:
    """Per-component quantities the E-step needs ([LP-GMM] 3.1, Preprocess)."""
    logdet: np.ndarray              # [K] log |C_k| (of the ridged C_k for "full")
    chol: np.ndarray | None = None  # [K, D, D] lower Cholesky factors ("full")
    ridge: np.ndarray | None = None  # [K] eps actually added ("full")
    retries: np.ndarray | None = None  # [K] ridge escalations needed ("full")


@dataclass
class StepResult:
    """Everything one EM iteration produces."""
    ll: float                # sum_n lse_n under the input parameters
    nk: np.ndarray           # [K]  s0 = sum_n G_nk
    s1: np.ndarray           # [K, D] sum_n G_nk x_n
    s2: np.ndarray           # raw second moments: [K,D] sum G x^2 (diag),
                             # [K] sum G |x|^2 (iso), [K,D,D] sum G x x^T (full)
    params: Params           # theta after the M-step
    prepared: Prepared = field(repr=False, default=None)


# ----------------------------------------------------------------------------
# Preprocess: log-determinants and Cholesky factors.  [LP-GMM] 1.2 (route 2,
# Cholesky: Sigma = L L^T, |Sigma| = (prod L_ii)^2), 3.1 (Preprocess kernel),
# 4.1 (ridge Sigma + eps I before the factorisation).
# ----------------------------------------------------------------------------

def cholesky_lower(a: np.ndarray) -> np.ndarray:
    """Textbook Cholesky-Banachiewicz factorisation A = L L^T, row by row.

    Raises NotPositiveDefinite on the first non-positive pivot.
    """
    n = a.shape[0]
    L = np.zeros_like(a, dtype=np.float64)
    for i in range(n):
        for j in range(i + 1):
            s = a[i, j] - float(np.dot(L[i, :j], L[j, :j]))
            if i == j:
                if not s > 0.0:
                    raise NotPositiveDefinite(f"pivot {i} = {s}")
                L[i, i] = math.sqrt(s)
            else:
                L[i, j] = s / L[j, j]
    return L


def ridged_cholesky(cov: np.ndarray, ridge_rel: float):
    """Factor C + eps I with eps = ridge_rel * |trace(C)| / D ([LP-GMM] 4.1).

    The ridge is always added.  If a pivot fails, eps becomes
    max(10 eps, 1e-3 |trace(C)| / D) and the factorisation is retried, at
    most RIDGE_RETRIES times; after that the covariance is reported as not
    positive definite.  Returns (L, eps, retries).
    """
    d = cov.shape[0]
    scale = abs(float(np.trace(cov))) / d
    eps = ridge_rel * scale
    for attempt in range(RIDGE_RETRIES + 1):
        try:
            L = cholesky_lower(cov + eps * np.eye(d))
            return L, eps, attempt
        except NotPositiveDefinite:
            eps = max(10.0 * eps, DEFAULT_RIDGE_REL * scale)
    raise NotPositiveDefinite("covariance not positive definite after ridge retries")


def prepare(p: Params, ridge_rel: float = DEFAULT_RIDGE_REL) -> Prepared:
    """Per-component log|C_k| (and L_k for full covariance)."""
    K, D = p.k, p.d
    if p.cov_type == "diag":
        return Prepared(logdet=np.sum(np.log(p.cov), axis=1))
    if p.cov_type == "iso":
        return Prepared(logdet=D * np.log(p.cov))
    chol = np.zeros((K, D, D))
    ridge = np.zeros(K)
    retries = np.zeros(K, dtype=np.int64)
    for k in range(K):
        chol[k], ridge[k], retries[k] = ridged_cholesky(p.cov[k], ridge_rel)
    logdet = 2.0 * np.sum(np.log(np.diagonal(chol, axis1=1, axis2=2)), axis=1)
    return Prepared(logdet=logdet, chol=chol, ridge=ridge, retries=retries)


def forward_substitution(L: np.ndarray, R: np.ndarray) -> np.ndarray:
    """Solve L z_n = r_n for every row r_n of R (column sweep).

    [LP-GMM] 1.2: z = L^{-1}(x - mu) by a triangular solve, no inverse.
    """
    Z = np.array(R, dtype=np.float64, copy=True)
    D = L.shape[0]
    for j in range(D):
        Z[:, j] /= L[j, j]
        if j + 1 < D:
            Z[:, j + 1:] -= np.outer(Z[:, j], L[j + 1:, j])
    return Z


# ----------------------------------------------------------------------------
# E-step.  [LP-GMM] 1.1 (posterior p(z=k|x) = pi_k N_k / sum_j pi_j N_j),
# 1.2 (multivariate density), 4.2 (log-space posterior with max shift).
# ----------------------------------------------------------------------------

def sq_mahalanobis(x: np.ndarray, p: Params, prep: Prepared) -> np.ndarray:
    """d2[n, k] = (x_n - mu_k)^T C_k^{-1} (x_n - mu_k), centred form."""
    n = x.shape[0]
    out = np.empty((n, p.k))
    for k in range(p.k):
        r = x - p.mu[k]
        if p.cov_type == "diag":
            out[:, k] = np.sum(r * r / p.cov[k], axis=1)
        elif p.cov_type == "iso":
            out[:, k] = np.sum(r * r, axis=1) / p.cov[k]
        else:
            z = forward_substitution(prep.chol[k], r)
            out[:, k] = np.sum(z * z, axis=1)
    return out


def log_joint(x: np.ndarray, p: Params, prep: Prepared) -> np.ndarray:
    """a[n, k] = log pi_k + log N(x_n | mu_k, C_k).

    log N = -1/2 (D log 2pi + log|C_k| + d2_nk).  log 0 = -inf is allowed for
    a zero weight.
    """
    d2 = sq_mahalanobis(x, p, prep)
    with np.errstate(divide="ignore"):
        log_pi = np.log(p.pi)
    return log_pi[None, :] - 0.5 * (p.d * LOG_2PI + prep.logdet[None, :] + d2)


def log_normaliser(a: np.ndarray) -> np.ndarray:
    """lse_n = m_n + log sum_k exp(a_nk - m_n), m_n = max_k a_nk."""
    m = np.max(a, axis=1)
    return m + np.log(np.sum(np.exp(a - m[:, None]), axis=1))


def responsibilities(a: np.ndarray, lse: np.ndarray) -> np.ndarray:
    """G_nk = exp(a_nk - lse_n); every row sums to 1."""
    return np.exp(a - lse[:, None])


def _chunks(n: int, chunk: int):
    for lo in range(0, n, chunk):
        yield lo, min(n, lo + chunk)


def loglik(x: np.ndarray, p: Params, ridge_rel: float = DEFAULT_RIDGE_REL,
           chunk: int = CHUNK):
    """E-step only ([LP-GMM] 1.1: inference needs just the E-step).

    Returns (LL, lse[N], argmax[N]); argmax takes the lowest k on ties.
    """
    x = np.asarray(x, dtype=np.float64)
    prep = prepare(p, ridge_rel)
    lse = np.empty(x.shape[0])
    arg = np.empty(x.shape[0], dtype=np.int64)
    for lo, hi in _chunks(x.shape[0], chunk):
        a = log_joint(x[lo:hi], p, prep)
        lse[lo:hi] = log_normaliser(a)
        arg[lo:hi] = np.argmax(a, axis=1)
    return float(np.sum(lse)), lse, arg


# ----------------------------------------------------------------------------
# M-step.  [Flash-GMM] Method, fused E-M step: s0 = sum gamma,
# s1 = sum gamma x, s2 = sum gamma x x^T; parameters updated from them after
# one pass.  The oracle takes the plain two-pass route (mean first, then the
# covariance centred about it) instead of s2/s0 - mu^2.
# ----------------------------------------------------------------------------

def em_step(x: np.ndarray, p: Params, var_floor: float = DEFAULT_VAR_FLOOR,
            ridge_rel: float = DEFAULT_RIDGE_REL, chunk: int = CHUNK) -> StepResult:
    """One EM iteration from parameters p over points x ([N, D])."""
    x = np.asarray(x, dtype=np.float64)
    N, D = x.shape
    K = p.k
    if D != p.d:
        raise ValueError("dimension mismatch")
    prep = prepare(p, ridge_rel)

    # pass 1: E-step, LL, N_k, first and raw second moments
    ll = 0.0
    nk = np.zeros(K)
    s1 = np.zeros((K, D))
    s2 = np.zeros({"diag": (K, D), "iso": (K,), "full": (K, D, D)}[p.cov_type])
    for lo, hi in _chunks(N, chunk):
        xc = x[lo:hi]
        a = log_joint(xc, p, prep)
        lse = log_normaliser(a)
        g = responsibilities(a, lse)
        ll += float(np.sum(lse))
        nk += np.sum(g, axis=0)
        s1 += g.T @ xc
        if p.cov_type == "diag":
            s2 += g.T @ (xc * xc)
        elif p.cov_type == "iso":
            s2 += g.T @ np.sum(xc * xc, axis=1)
        else:
            for k in range(K):
                s2[k] += (g[:, k:k + 1] * xc).T @ xc

    empty = nk < EMPTY_NK
    safe_nk = np.where(empty, 1.0, nk)
    mu_new = np.where(empty[:, None], p.mu, s1 / safe_nk[:, None])

    # pass 2: covariance centred about the new mean (responsibilities recomputed)
    if p.cov_type == "full":
        acc = np.zeros((K, D, D))
    elif p.cov_type == "diag":
        acc = np.zeros((K, D))
    else:
        acc = np.zeros(K)
    for lo, hi in _chunks(N, chunk):
        xc = x[lo:hi]
        a = log_joint(xc, p, prep)
        g = responsibilities(a, log_normaliser(a))
        for k in range(K):
            r = xc - mu_new[k]
            if p.cov_type == "diag":
                acc[k] += g[:, k] @ (r * r)
            elif p.cov_type == "iso":
                acc[k] += g[:, k] @ np.sum(r * r, axis=1)
            else:
                acc[k] += (g[:, k:k + 1] * r).T @ r

    if p.cov_type == "diag":
        cov_new = np.maximum(acc / safe_nk[:, None], var_floor)
        cov_new = np.where(empty[:, None], p.cov, cov_new)
    elif p.cov_type == "iso":
        cov_new = np.maximum(acc / (D * safe_nk), var_floor)
        cov_new = np.where(empty, p.cov, cov_new)
    else:
        cov_new = acc / safe_nk[:, None, None]
        cov_new = np.where(empty[:, None, None], p.cov, cov_new)
    pi_new = nk / N
    return StepResult(ll=ll, nk=nk, s1=s1, s2=s2,
                      params=Params(pi_new, mu_new, cov_new, p.cov_type),
                      prepared=prep)


def fit(x: np.ndarray, p: Params, iters: int, var_floor: float = DEFAULT_VAR_FLOOR,
        ridge_rel: float = DEFAULT_RIDGE_REL, chunk: int = CHUNK):
    """`iters` EM iterations; returns (list of LL per iteration, final params).

    The iteration count is fixed by the caller ([Flash-GMM] Method, outputs:
    the kernel is called repeatedly until LL converges or an iteration cap).
    """
    lls = []
    for _ in range(iters):
        r = em_step(x, p, var_floor, ridge_rel, chunk)
        lls.append(r.ll)
        p = r.params
    return lls, p
