"""Helpers for the GPU parity tests: device copies, margin-guaranteed inputs (via the oracle)."""
from __future__ import annotations

import numpy as np

import moe_inputs as mi
import oracle


def dev(a: np.ndarray, device="cuda"):
    """numpy -> torch device tensor; uint16 arrays are bf16 bit patterns."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def host(t) -> np.ndarray:
    """torch tensor -> numpy; bf16 comes back as float64 values."""
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.float().numpy().astype(np.float64)
    return t.numpy()


def sorted_gaps(l64: np.ndarray, k: int) -> np.ndarray:
    """Per row: the smallest gap between consecutive entries among the k+1 largest logits."""
    E = l64.shape[1]
    s = -np.sort(-l64, axis=1)[:, : min(k + 1, E)]
    if s.shape[1] < 2:
        return np.full(l64.shape[0], np.inf)
    return np.min(s[:, :-1] - s[:, 1:], axis=1)


def margin_x(spec, layer: int = 0, tau_rel: float = 1e-3, b=None, max_rounds: int = 50):
    """Token rows whose oracle fp64 logits keep every gap among the k+1 largest above
    tau_rel * rms(row), so the selection and its order are decided identically by any
    fp32 summation order whose error stays below half that gap.  Violating rows are
    redrawn from the next attempt of their own sub-stream."""
    wr, b0 = mi.host_router(spec, layer)
    b = b0 if b is None else b
    attempts = np.zeros(spec.T, np.int64)
    x = mi.host_x(spec, layer, attempts)
    _, l64 = oracle.router_logits(spec, x, wr, b)
    for _ in range(max_rounds):
        rms = np.sqrt(np.mean(l64 * l64, axis=1))
        bad = np.nonzero(sorted_gaps(l64, spec.k) < tau_rel * rms)[0]
        if bad.size == 0:
            return x, wr, b, attempts
        attempts[bad] += 1
        x[bad] = mi.host_x(spec, layer, attempts, rows=bad)
        _, l64[bad] = oracle.router_logits(spec, np.ascontiguousarray(x[bad]), wr, b)
    raise RuntimeError("could not draw margin-guaranteed tokens")
