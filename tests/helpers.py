"""Shared helpers for the parity tests (tolerance check, device transfer)."""
import numpy as np

RTOL, ATOL = 1e-4, 1e-6  # |gpu - oracle| <= RTOL * sum_k |w_k x_k| + ATOL per element


def tol_ratio(y_gpu, y_ref, a):
    """Per-element |gpu - oracle| / (RTOL * a + ATOL), computed in fp64."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    return np.abs(y_gpu - y_ref) / (RTOL * np.asarray(a) + ATOL)


def assert_within_tol(y_gpu, y_ref, a, what=""):
    r = tol_ratio(y_gpu, y_ref, a)
    bad = ~(r <= 1.0)  # NaN counts as bad
    if bad.any():
        idx = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} of {r.size} outside tolerance; first at {tuple(idx)}: "
                             f"gpu={np.asarray(y_gpu)[tuple(idx)]!r} oracle={y_ref[tuple(idx)]!r} "
                             f"a={np.asarray(a)[tuple(idx)]!r}; max ratio {np.nanmax(r):.3g}")
    return float(r.max()) if r.size else 0.0
