"""Writes tests/golden/oracle_tiny.json: a small seeded problem and the
oracle's answer, a regression fixture for the oracle itself.  Calls only
oracle/ (and numpy to draw the seeded inputs)."""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402


def problem(cov_type):
    rng = np.random.Generator(np.random.PCG64(77))
    n, d, k = 48, 3, 2
    x = np.round(rng.standard_normal((n, d)) * 2.0 + np.repeat([[0, 0, 0], [4, 1, -3]], n // 2, axis=0), 3)
    mu = np.array([[0.5, 0.0, 0.2], [3.0, 1.5, -2.0]])
    pi = np.array([0.4, 0.6])
    cov = {"diag": np.array([[1.0, 2.0, 0.5], [1.5, 1.0, 1.0]]),
           "iso": np.array([1.0, 2.0]),
           "full": np.array([[[2.0, 0.3, 0.0], [0.3, 1.0, 0.2], [0.0, 0.2, 1.5]],
                             [[1.0, -0.4, 0.1], [-0.4, 2.0, 0.0], [0.1, 0.0, 0.7]]])}[cov_type]
    return x, oracle.Params(pi, mu, cov, cov_type)


def main():
    out = {"_about": "oracle regression fixture; regenerate with make_golden.py"}
    for ct in ("diag", "iso", "full"):
        x, p = problem(ct)
        r = oracle.em_step(x, p)
        out[ct] = {"x": x.tolist(), "pi": p.pi.tolist(), "mu": p.mu.tolist(), "cov": p.cov.tolist(),
                   "ll": r.ll, "pi_new": r.params.pi.tolist(), "mu_new": r.params.mu.tolist(),
                   "cov_new": r.params.cov.tolist()}
    with open(os.path.join(HERE, "oracle_tiny.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
