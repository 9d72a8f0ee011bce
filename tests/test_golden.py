"""Golden fixtures: the pages' printed numbers, and the oracle regression file."""
import json
import os

import numpy as np
import torch

import oracle

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def facts():
    with open(os.path.join(HERE, "page_facts.json")) as f:
        return json.load(f)


def test_page_facts_fp_ranges():
    f = facts()
    assert float(np.finfo(np.float16).max) == f["fp16_max"]["value"]
    e32 = float(torch.exp(torch.tensor(-50.0, dtype=torch.float32)))
    assert abs(e32 - f["exp_minus_50_fp32"]["value"]) <= f["exp_minus_50_fp32"]["rel_tol"] * 1.9e-22
    assert float(torch.tensor(e32).to(torch.float16)) == 0.0
    assert oracle.DEFAULT_RIDGE_REL == f["ridge_rel"]["value"]


def test_oracle_regression_fixture():
    with open(os.path.join(HERE, "oracle_tiny.json")) as f:
        g = json.load(f)
    for ct in ("diag", "iso", "full"):
        c = g[ct]
        p = oracle.Params(np.array(c["pi"]), np.array(c["mu"]), np.array(c["cov"]), ct)
        r = oracle.em_step(np.array(c["x"]), p)
        np.testing.assert_allclose(r.ll, c["ll"], rtol=1e-13)
        np.testing.assert_allclose(r.params.pi, c["pi_new"], rtol=1e-12)
        np.testing.assert_allclose(r.params.mu, c["mu_new"], rtol=1e-12)
        np.testing.assert_allclose(r.params.cov, c["cov_new"], rtol=1e-12)
