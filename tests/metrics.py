"""Error metrics used by the parity tests (operator-debugging article,
section 3.2: relative error, max-abs error, percentiles, cosine)."""
import numpy as np


def rel_inf(a, ref):
    """||a - ref||_inf / ||ref||_inf (per-tensor gate for parameters)."""
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(a - ref)) / den) if den > 0 else float(np.max(np.abs(a - ref)))


def rel(a, ref):
    return abs(float(a) - float(ref)) / abs(float(ref)) if ref != 0 else abs(float(a))


def cosine(a, ref):
    a = np.ravel(np.asarray(a, dtype=np.float64))
    ref = np.ravel(np.asarray(ref, dtype=np.float64))
    return float(a @ ref / (np.linalg.norm(a) * np.linalg.norm(ref)))


def percentiles(a, ref, eps=1e-30):
    e = np.abs(np.asarray(a, np.float64) - np.asarray(ref, np.float64)) / (np.abs(ref) + eps)
    return {q: float(np.percentile(e, q)) for q in (50, 95, 99)}
