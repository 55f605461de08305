"""Shared test helpers: tolerance checks and small numpy utilities (no layer arithmetic)."""
from __future__ import annotations

import numpy as np


def bf16_to_f64(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    with np.errstate(invalid="ignore"):
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return bf16_to_f64(a)
    return a.astype(np.float64)


def tol_violations(got, ref, rel: float = 2e-2, abs_of_rms: float = 1e-2, eps: float = 1e-30):
    """Element-wise bound |got - ref| <= abs_of_rms * max(rms(ref), eps) + rel * |ref|.

    NaN must sit at the same positions in both; +-inf must match exactly.
    Returns (n_bad, max_abs_err, max_rel_err, bound_rms).
    """
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    nan_g, nan_r = np.isnan(got), np.isnan(ref)
    bad_nan = int(np.sum(nan_g != nan_r))
    inf_r = np.isinf(ref)
    bad_inf = int(np.sum(inf_r & (got != ref)))
    fin = ~(nan_r | inf_r | nan_g)
    r = ref[fin]
    g = got[fin]
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    bound = abs_of_rms * max(rms, eps) + rel * np.abs(r)
    err = np.abs(g - r)
    bad = int(np.sum(err > bound)) + bad_nan + bad_inf
    max_abs = float(err.max()) if err.size else 0.0
    sig = np.abs(r) >= 1e-3 * max(rms, eps)
    max_rel = float((err[sig] / np.abs(r[sig])).max()) if np.any(sig) else 0.0
    return bad, max_abs, max_rel, rms


def assert_close(got, ref, rel: float = 2e-2, abs_of_rms: float = 1e-2, what: str = ""):
    bad, max_abs, max_rel, rms = tol_violations(got, ref, rel, abs_of_rms)
    assert bad == 0, (f"{what}: {bad} elements outside |d| <= {abs_of_rms}*rms + {rel}*|ref| "
                      f"(max abs {max_abs:.3e}, max rel {max_rel:.3e}, rms {rms:.3e})")
    return max_abs, max_rel


def assert_literal(got, ref, what: str = ""):
    """The layer specification's bound read literally, |got - ref| <= 1e-2 + 2e-2 * |ref| (an
    absolute 1e-2), for workloads whose outputs are of order one (the bf16 128-expert layers);
    NaN positions must agree.  Prints the largest error relative to that bound."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape and np.array_equal(np.isnan(got), np.isnan(ref)), what
    fin = np.isfinite(ref)
    ratio = np.abs(got[fin] - ref[fin]) / (1e-2 + 2e-2 * np.abs(ref[fin]))
    worst = float(ratio.max()) if ratio.size else 0.0
    print(f"{what}: largest error / literal bound (1e-2 + 2e-2|ref|) {worst:.3e}", flush=True)
    assert worst <= 1.0, f"{what}: outside the literal bound 1e-2 + 2e-2*|ref| (ratio {worst:.3e})"


def ref_select(l: np.ndarray, k: int):
    """Brute-force selection: full stable sort of experts by (-logit, index) with NaN last."""
    E = len(l)
    def key(e):
        v = float(l[e])
        if np.isnan(v):
            return (1, 0.0, e)
        return (0, -v if v != 0.0 else 0.0, e)
    return sorted(range(E), key=key)[:k]
