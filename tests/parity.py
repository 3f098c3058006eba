"""Parity checks shared by the GPU tests: the relative L2 error over the
whole output (the page reports its errors this way), and an element-wise
bound next to it, so that an error confined to a few entries cannot hide in
the norm of a large output."""
import numpy as np

import oracle


def errors(x, ref):
    """(relative L2 error, largest entry error / rms of the reference)."""
    x, ref = np.asarray(x).ravel(), np.asarray(ref).ravel()
    rel = oracle.rel_l2(x, ref)
    rms = np.linalg.norm(ref) / np.sqrt(max(ref.size, 1))
    diff = np.abs(x - ref)
    worst = float(diff.max()) if diff.size else 0.0
    return rel, (worst / rms if rms > 0 else worst)


def within(x, ref, tol):
    """Relative L2 error <= tol, and every entry within 10 tol rms(ref) of
    the reference (NaN anywhere fails)."""
    rel, elem = errors(x, ref)
    return bool(np.isfinite(np.asarray(x)).all() and rel <= tol and elem <= 10 * tol), rel, elem
