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


def tile_boundary_tokens(idx: np.ndarray, E: int, T: int, n_shared: int, bm: int = 128) -> np.ndarray:
    """Tokens whose rows sit at the first or last sorted position of every m-tile of every expert
    (so every expert's first and last slot, and every ragged last tile, is among them), plus the
    shared expert's tile edges and the first and last token."""
    k = idx.shape[1]
    order = np.argsort(idx.reshape(-1), kind="stable")  # sorted position -> pair
    counts = np.bincount(idx.reshape(-1), minlength=E)
    offs = np.concatenate([[0], np.cumsum(counts)])
    pos = []
    for e in range(E):
        for m0 in range(offs[e], offs[e + 1], bm):
            pos += [m0, min(m0 + bm, offs[e + 1]) - 1]
    toks = set((order[np.array(pos, np.int64)] // k).tolist()) if pos else set()
    if n_shared:
        for m0 in range(0, T, bm):
            toks |= {m0, min(m0 + bm, T) - 1}
    toks |= {0, T - 1}
    return np.array(sorted(toks), np.int64)


def oracle_on_tokens(s, x, wr, b, tokens, flags: int = 0):
    """The oracle layer on the listed tokens (rows are independent), generating only the experts
    those tokens select: route with all E experts, evaluate the selected experts compacted.
    Returns the output and the compacted routing and weights it used."""
    xs = np.ascontiguousarray(x[tokens])
    l32s, _ = oracle.router_logits(s, xs, wr, b)
    idx_s, g_s = oracle.topk(s, l32s)
    need = sorted(set(idx_s.reshape(-1).tolist()))
    w = mi.host_experts(s, experts=need)
    sh = mi.host_experts(s, shared=True) if s.n_shared else None
    remap = np.full(s.E, -1, np.int64)
    remap[need] = np.arange(len(need))
    idx_c = remap[idx_s].astype(np.int32)
    sc = mi.LayerSpec(s.name, len(tokens), s.d, s.f, len(need), s.k, s.n_shared, s.f_shared, s.act, s.wt,
                      s.sigma_x, s.sigma_w, s.sigma_r)
    c, o, p, iv = oracle.permute(sc, idx_c)
    ys, ysh = oracle.grouped_ffn(sc, xs, p, o, w, sh, flags=flags)
    return dict(out=oracle.combine(sc, ys, iv, idx_c, g_s, ysh), spec=sc, xs=xs, idx=idx_s, idx_c=idx_c, g=g_s,
                perm=p, offsets=o, inv=iv, w=w, sh=sh, need=need)
