"""Checker self-test (operator-debugging article, section 7.2: check the
checker with deliberately wrong operators).  Each mutant is a copy of the
oracle with one plausible mistake planted in its source, on the CPU; the pin
suite must reject every one of them."""
import os
import sys
import types

import pytest

from tests import oracle_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "gmm_oracle.py")

MUTANTS = {
    "drop_log_pi": ("log_pi[None, :] - 0.5 *", "0.0 - 0.5 *"),
    "unbiased_variance": ("np.maximum(acc / safe_nk[:, None], var_floor)", "np.maximum(acc / (safe_nk[:, None] - 1.0), var_floor)"),
    "no_max_shift": ("return m + np.log(np.sum(np.exp(a - m[:, None]), axis=1))",
                     "return np.log(np.sum(np.exp(a), axis=1))"),
    "drop_dim_in_2pi": ("p.d * LOG_2PI", "LOG_2PI"),
    "half_logdet_full": ("logdet = 2.0 * np.sum(", "logdet = 1.0 * np.sum("),
    "transposed_factor": ("np.outer(Z[:, j], L[j + 1:, j])", "np.outer(Z[:, j], L[j, j + 1:])"),
    "swapped_s1_s2": ("s1 += g.T @ xc", "s1 += g.T @ (xc * xc)"),
    "rows_not_normalised": ("return np.exp(a - lse[:, None])", "return np.exp(a - lse[:, None] + 1e-3)"),
    "pi_over_n_plus_1": ("pi_new = nk / N", "pi_new = nk / (N + 1)"),
    "iso_missing_d": ("acc / (D * safe_nk)", "acc / safe_nk"),
    "centred_on_old_mean": ("r = xc - mu_new[k]", "r = xc - p.mu[k]"),
    "ridge_without_d": ("scale = abs(float(np.trace(cov))) / d", "scale = abs(float(np.trace(cov)))"),
    "sign_of_mahalanobis": ("- 0.5 * (p.d * LOG_2PI + prep.logdet[None, :] + d2)",
                            "- 0.5 * (p.d * LOG_2PI + prep.logdet[None, :] - d2)"),
    "iso_logdet_once": ("logdet=D * np.log(p.cov)", "logdet=np.log(p.cov)"),
    "floor_additive": ("np.maximum(acc / safe_nk[:, None], var_floor)",
                       "acc / safe_nk[:, None] + var_floor"),
}


def load_mutant(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    src = src.replace(old, new)
    modname = f"_oracle_mutant_{name}"
    mod = types.ModuleType(modname)
    mod.__file__ = SRC
    sys.modules[modname] = mod
    try:
        exec(compile(src, SRC, "exec"), mod.__dict__)
    except Exception:
        del sys.modules[modname]
        raise
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = load_mutant(name)
    failed = []
    try:
        for pin in oracle_pins.ALL_PINS:
            try:
                with _quiet():
                    pin(mod)
            except (AssertionError, FloatingPointError, ValueError, ZeroDivisionError,
                    mod.NotPositiveDefinite, OverflowError):
                failed.append(pin.__name__)
    finally:
        sys.modules.pop(mod.__name__, None)
    assert failed, f"mutant {name} passed every pin"


class _quiet:
    def __enter__(self):
        import warnings
        import numpy as np
        self._w = warnings.catch_warnings()
        self._w.__enter__()
        warnings.simplefilter("ignore")
        self._e = np.errstate(all="ignore")
        self._e.__enter__()

    def __exit__(self, *a):
        self._e.__exit__(*a)
        self._w.__exit__(*a)
        return False


# ---- the assignment / start / fit-loop module --------------------------------
SRC_AF = os.path.join(os.path.dirname(SRC), "gmm_assign_fit.py")
MUTANTS_AF = {
    "topm_ties_high_index_first": ("np.lexsort((ks, -a[i]))", "np.lexsort((-ks, -a[i]))"),
    "topm_ascending": ("np.lexsort((ks, -a[i]))", "np.lexsort((ks, a[i]))"),
    "topm_gamma_without_lse": ("np.exp(a[i, order] - lse[i])", "np.exp(a[i, order])"),
    "floyd_range_off_by_one": ("t = r % (j + 1)", "t = r % j if j else 0"),
    "floyd_keeps_duplicate_draw": ("chosen.add(j if t in chosen else t)", "chosen.add(t)"),
    "splitmix_shift": ("z = ((z ^ (z >> 30))", "z = ((z ^ (z >> 31))"),
    "splitmix_no_increment": ("state = (state + GOLDEN) & MASK64", "state = state & MASK64"),
    "fit_tolerance_not_per_point": ("abs(lls[-1] - lls[-2]) / n < tol", "abs(lls[-1] - lls[-2]) < tol"),
    "fit_returns_previous_params": ("        p = r.params\n        if len(lls)", "        if len(lls)"),
    "start_half_variance": ('"diag": np.ones((k, d)), "iso"', '"diag": 0.5 * np.ones((k, d)), "iso"'),
}


def load_mutant_af(name):
    old, new = MUTANTS_AF[name]
    src = open(SRC_AF).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    src = src.replace(old, new).replace("from .gmm_oracle import", "from oracle.gmm_oracle import")
    modname = f"_oracle_af_mutant_{name}"
    mod = types.ModuleType(modname)
    mod.__file__ = SRC_AF
    sys.modules[modname] = mod
    try:
        exec(compile(src, SRC_AF, "exec"), mod.__dict__)
    except Exception:
        del sys.modules[modname]
        raise
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS_AF))
def test_assign_fit_mutant_is_caught(name):
    import oracle
    from tests import oracle_pins_assign_fit as P
    mod = load_mutant_af(name)
    failed = []
    try:
        for pin in P.ALL_PINS:
            try:
                with _quiet():
                    pin(mod, oracle.gmm_oracle)
            except (AssertionError, FloatingPointError, ValueError, ZeroDivisionError, OverflowError,
                    IndexError):
                failed.append(pin.__name__)
    finally:
        sys.modules.pop(mod.__name__, None)
    assert failed, f"mutant {name} passed every pin"
