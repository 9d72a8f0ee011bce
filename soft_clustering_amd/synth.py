"""Seeded synthetic Gaussian-mixture workloads.

This module only draws inputs: a ground-truth mixture, points sampled from it
(stored as fp32, fp16 or bf16 with round-to-nearest-even), and the EM starting
parameters.  It holds none of the EM arithmetic, so both the HIP path and the
CPU oracle can be fed from it without sharing any of the method's code.

The workloads mirror the pages' scales: the low-precision operator write-up
measures D = 32..64, K = 8..32 (section 2.3) and the Flash-GMM summary targets
up to 1e9 points x 1024 components on one device (Problem section).  No public
dataset is named there, so seeded mixtures stand in for them.

Recipe (all randomness seeded):
  1. pi ~ Dirichlet(1_K); means and covariances from the workload's spec;
  2. z_n ~ Categorical(pi) i.i.d.;
  3. x_n = mu_{z_n} + noise with the covariance of component z_n;
  4. cast to the storage dtype (round to nearest even).
Parameters come from numpy PCG64(data_seed); the bulk points from a torch
generator on the target device seeded with data_seed, consumed in fixed
2^20-row chunks, so X depends only on (workload, seed, device type).
The EM start is K distinct data points (drawn with PCG64(init_seed)) as
means, unit variances (identity for full covariance) and pi = 1/K.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass

import numpy as np

CHUNK_ROWS = 1 << 20


@dataclass(frozen=True)
class Workload:
    name: str
    n: int
    d: int
    k: int
    cov: str            # "diag" | "iso" | "full"
    x_dtype: str        # "f32" | "bf16" | "f16"
    means: tuple        # ("uniform", lo, hi) | ("normal", scale)
    var: tuple          # ("uniform", lo, hi) | ("loguniform", lo, hi) | ("eig_log10", lo, hi)
    iters: int = 1
    data_seed: int = 1000
    init_seed: int = 2000

    def with_n(self, n: int, suffix: str = "") -> "Workload":
        return Workload(self.name + suffix, n, self.d, self.k, self.cov, self.x_dtype,
                        self.means, self.var, self.iters, self.data_seed, self.init_seed)

    @property
    def x_bytes(self) -> int:
        return self.n * self.d * (4 if self.x_dtype == "f32" else 2)


WORKLOADS = {
    w.name: w for w in [
        Workload("diag-f32-n4096-d16-k8", 4096, 16, 8, "diag", "f32",
                 ("uniform", -10.0, 10.0), ("uniform", 0.5, 2.0), iters=10,
                 data_seed=1001, init_seed=2001),
        Workload("diag-f32-n1e6-d64-k16", 1_000_000, 64, 16, "diag", "f32",
                 ("normal", 5.0), ("uniform", 0.5, 2.0), iters=20,
                 data_seed=1002, init_seed=2002),
        Workload("iso-bf16-n1e7-d128-k256", 10_000_000, 128, 256, "iso", "bf16",
                 ("normal", 3.0), ("uniform", 0.25, 1.0), iters=1,
                 data_seed=1003, init_seed=2003),
        Workload("diag-bf16-n2e8-d128-k1024", 200_000_000, 128, 1024, "diag", "bf16",
                 ("normal", 2.0), ("loguniform", 0.1, 2.0), iters=1,
                 data_seed=1004, init_seed=2004),
        Workload("full-f16-n1e6-d64-k16", 1_000_000, 64, 16, "full", "f16",
                 ("normal", 5.0), ("eig_log10", -1.5, 1.5), iters=1,
                 data_seed=1005, init_seed=2005),
        # the full-covariance mixture at D = 128 (the widest D the library takes)
        Workload("full-f16-n1e6-d128-k16", 1_000_000, 128, 16, "full", "f16",
                 ("normal", 5.0), ("eig_log10", -1.5, 1.5), iters=1,
                 data_seed=1006, init_seed=2006),
    ]
}


@dataclass
class Mixture:
    """Ground truth: pi [K], mu [K, D], cov as [K, D] / [K] / [K, D, D];
    for full covariance also its eigen-decomposition (q [K,D,D], lam [K,D])."""
    pi: np.ndarray
    mu: np.ndarray
    cov: np.ndarray
    q: np.ndarray | None = None
    lam: np.ndarray | None = None


def _haar_orthogonal(rng: np.random.Generator, d: int) -> np.ndarray:
    """Haar-distributed orthogonal matrix: QR of a Gaussian, signs fixed."""
    a = rng.standard_normal((d, d))
    q, r = np.linalg.qr(a)
    return q * np.sign(np.diag(r))[None, :]


def make_mixture(w: Workload, seed: int | None = None) -> Mixture:
    rng = np.random.Generator(np.random.PCG64(w.data_seed if seed is None else seed))
    K, D = w.k, w.d
    pi = rng.dirichlet(np.ones(K))
    if w.means[0] == "uniform":
        mu = rng.uniform(w.means[1], w.means[2], size=(K, D))
    else:
        mu = w.means[1] * rng.standard_normal((K, D))
    kind, lo, hi = w.var
    if w.cov == "full":
        q = np.stack([_haar_orthogonal(rng, D) for _ in range(K)])
        lam = 10.0 ** rng.uniform(lo, hi, size=(K, D))
        cov = np.einsum("kij,kj,klj->kil", q, lam, q)
        cov = 0.5 * (cov + np.transpose(cov, (0, 2, 1)))
        return Mixture(pi, mu, cov, q, lam)
    shape = (K, D) if w.cov == "diag" else (K,)
    if kind == "uniform":
        cov = rng.uniform(lo, hi, size=shape)
    elif kind == "loguniform":
        cov = np.exp(rng.uniform(np.log(lo), np.log(hi), size=shape))
    else:
        raise ValueError(kind)
    return Mixture(pi, mu, cov)


def torch_dtype(x_dtype: str):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[x_dtype]


def sample_points(w: Workload, mix: Mixture, device="cpu", n: int | None = None,
                  seed: int | None = None, ldx: int | None = None):
    """Draw n points from the mixture as a torch tensor [n, D] (or a strided
    view of an [n, ldx] buffer) in the storage dtype on `device`."""
    import torch
    n = w.n if n is None else n
    D = w.d
    ldx = D if ldx is None else ldx
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.data_seed if seed is None else seed)
    buf = torch.zeros((n, ldx), dtype=torch_dtype(w.x_dtype), device=dev)
    pi = torch.tensor(mix.pi, dtype=torch.float64, device=dev)
    mu = torch.tensor(mix.mu, dtype=torch.float32, device=dev)
    if w.cov == "full":
        scale = torch.tensor(np.sqrt(mix.lam), dtype=torch.float32, device=dev)
        qt = torch.tensor(np.transpose(mix.q, (0, 2, 1)).copy(), dtype=torch.float32, device=dev)
    else:
        sd = torch.tensor(np.sqrt(mix.cov), dtype=torch.float32, device=dev)
    for lo in range(0, n, CHUNK_ROWS):
        m = min(CHUNK_ROWS, n - lo)
        z = torch.multinomial(pi, m, replacement=True, generator=gen)
        eps = torch.randn((m, D), generator=gen, device=dev, dtype=torch.float32)
        if w.cov == "diag":
            x = mu[z] + eps * sd[z]
        elif w.cov == "iso":
            x = mu[z] + eps * sd[z][:, None]
        else:
            x = torch.empty((m, D), dtype=torch.float32, device=dev)
            for k in range(w.k):
                idx = (z == k).nonzero().flatten()
                if idx.numel():
                    x[idx] = mu[k] + (eps[idx] * scale[k]) @ qt[k]
        buf[lo:lo + m, :D] = x.to(buf.dtype)
    return buf[:, :D]


def init_params(w: Workload, x, seed: int | None = None):
    """EM start: K distinct data points as means, unit (co)variances, pi=1/K.

    x is the stored point tensor (any device); returns numpy fp32 arrays
    (pi [K], mu [K, D], cov) with cov shaped for w.cov."""
    import torch
    n = x.shape[0]
    rng = np.random.Generator(np.random.PCG64(w.init_seed if seed is None else seed))
    k = w.k
    idx = np.sort(rng.choice(n, size=k, replace=False)) if k <= n else \
        rng.choice(n, size=k, replace=True)
    mu = x[torch.as_tensor(idx, device=x.device)].to(torch.float32).cpu().numpy()
    pi = np.full(k, 1.0 / k, dtype=np.float32)
    if w.cov == "diag":
        cov = np.ones((k, w.d), dtype=np.float32)
    elif w.cov == "iso":
        cov = np.ones(k, dtype=np.float32)
    else:
        cov = np.tile(np.eye(w.d, dtype=np.float32), (k, 1, 1))
    return pi, np.ascontiguousarray(mu, dtype=np.float32), cov


def sha256_of(x) -> str:
    """Hash of the stored bytes of X (for failure replay)."""
    import torch
    h = hashlib.sha256()
    t = x.contiguous()
    step = CHUNK_ROWS
    for lo in range(0, t.shape[0], step):
        h.update(t[lo:lo + step].cpu().view(torch.uint8).numpy().tobytes())
    return h.hexdigest()
