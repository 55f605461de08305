"""Seeded synthetic inputs for the routed mixture-of-experts layer.

This package generates inputs only; it holds none of the layer's arithmetic.
Both the CPU oracle's tests and the GPU path's tests/bench draw from it, so
the two sides see the same bytes.

Generator (defined in gen_host.c, mirrored on the device in gen_device.hip):
counter-based SplitMix64 words, Irwin-Hall "normal" values (sum of four
16-bit uniforms, std sigma, bounded at +-3.46 sigma, exact integer work and one
fp32 multiply) and bf16 by round-to-nearest-even.  Every tensor has its own
sub-stream key derive(derive(derive(root(seed), layer), tag), sub), where
`sub` is the expert index for per-expert tensors and (attempt << 32) | t for
token row t of x, so single experts or single rows can be regenerated alone.

Workload shapes follow the layer sizes the pages give: DeepSeek-V4-Flash
routes 6 of 256 experts in each of 43 layers at FP4 precision (dothoosh.com
FreeToken article, "FreeToken architecture and the sparsity puzzle"; aihot.vn
FreeToken article, "The gap it targets"), and Gemma 4 26B A4B routes 8 of 128
experts plus one shared expert (dothoosh.com TurboFieldfare article,
"Background: Gemma 4 26B A4B").  The remaining sizes (d_model, d_ff, value
distributions) are this project's stated synthetic choices.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, replace
from typing import Iterable, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libmoe_gen_host.so")
DEV_LIB = os.path.join(_HERE, "libmoe_gen_dev.so")

GAMMA = 0x9E3779B97F4A7C15
MASK64 = (1 << 64) - 1

# Sub-stream tags.
TAG_X, TAG_WR, TAG_W13, TAG_W2, TAG_S13, TAG_S2, TAG_W13S, TAG_W2S, TAG_S13S, TAG_S2S, TAG_H0, TAG_PERM = range(1, 13)

IRWIN_HALL_STD = math.sqrt((2.0 ** 32 - 1.0) / 3.0)

_host = None
_dev = None


def _load_host():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            raise RuntimeError(f"{HOST_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(HOST_LIB)
        u64, i64, f32 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_float
        vp, ci = ctypes.c_void_p, ctypes.c_int
        lib.mg_derive.restype = u64
        lib.mg_derive.argtypes = [u64, u64]
        lib.mg_word.restype = u64
        lib.mg_word.argtypes = [u64, u64]
        lib.mg_fill_normal_f32.argtypes = [vp, i64, u64, f32, i64]
        lib.mg_fill_normal_bf16.argtypes = [vp, i64, u64, f32, i64]
        lib.mg_fill_bytes.argtypes = [vp, i64, u64, i64]
        lib.mg_fill_scale_bytes.argtypes = [vp, i64, u64, ci, ci, i64]
        lib.mg_fill_normal_bf16_experts.argtypes = [vp, i64, i64, i64, u64, f32]
        lib.mg_fill_normal_f32_experts.argtypes = [vp, i64, i64, i64, u64, f32]
        lib.mg_fill_bytes_experts.argtypes = [vp, i64, i64, i64, u64]
        lib.mg_fill_scale_bytes_experts.argtypes = [vp, i64, i64, i64, u64, ci, ci]
        _host = lib
    return _host


def _load_dev():
    global _dev
    if _dev is None:
        import torch  # noqa: F401  -- bind the library to torch's HIP runtime (loaded first)
        if not os.path.exists(DEV_LIB):
            raise RuntimeError(f"{DEV_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(DEV_LIB)
        u64, i64, f32 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_float
        vp, ci = ctypes.c_void_p, ctypes.c_int
        lib.mgd_fill_normal_bf16.argtypes = [vp, i64, i64, i64, u64, f32, ci, vp]
        lib.mgd_fill_normal_f32.argtypes = [vp, i64, i64, i64, u64, f32, ci, vp]
        lib.mgd_fill_bytes.argtypes = [vp, i64, i64, i64, u64, ci, vp]
        lib.mgd_fill_scale_bytes.argtypes = [vp, i64, i64, i64, u64, ci, ci, ci, vp]
        for fn in (lib.mgd_fill_normal_bf16, lib.mgd_fill_normal_f32, lib.mgd_fill_bytes, lib.mgd_fill_scale_bytes):
            fn.restype = ctypes.c_int
        _dev = lib
    return _dev


def derive(key: int, x: int) -> int:
    return int(_load_host().mg_derive(int(key) & MASK64, int(x) & MASK64))


def word(key: int, i: int) -> int:
    return int(_load_host().mg_word(int(key) & MASK64, int(i) & MASK64))


def root(seed: int) -> int:
    return derive(seed, 0)


def tensor_key(seed: int, layer: int, tag: int) -> int:
    return derive(derive(root(seed), layer), tag)


def normal_scale(sigma: float) -> float:
    """fp32 multiplier c turning an Irwin-Hall integer into a value of std sigma."""
    return float(np.float32(sigma / IRWIN_HALL_STD))


# ----------------------------------------------------------------------------------------------
# Workload specifications
# ----------------------------------------------------------------------------------------------
@dataclass(frozen=True)
class LayerSpec:
    name: str
    T: int
    d: int            # d_model
    f: int            # routed expert d_ff
    E: int            # routed experts
    k: int            # top-k
    n_shared: int     # 0 or 1 always-on shared expert
    f_shared: int
    act: str          # 'f32' | 'bf16'
    wt: str           # 'f32' | 'bf16' | 'mxfp4' | 'nvfp4'
    sigma_x: float
    sigma_w: float
    sigma_r: float
    bias: str = "zero"   # 'zero' | 'zipf'
    scale_lo: int = 119  # scale byte range: MXFP4 E8M0 119..127 = 2^-8 .. 2^0 (NVFP4 E4M3: 0x20..0x3F)
    scale_hi: int = 127
    seed: int = 1000
    n_layers: int = 1

    def with_T(self, T: int) -> "LayerSpec":
        return replace(self, T=T)


CONFIGS = {
    # Tiny fp32 layer.
    "c0": LayerSpec("c0", 16, 256, 128, 8, 2, 0, 0, "f32", "f32", 0.02, 0.02, 0.02, seed=1000),
    # Decode, bf16, 128 routed top-8 + 1 shared (Gemma-4-26B-A4B-like routing).
    "c1": LayerSpec("c1", 1, 2048, 768, 128, 8, 1, 768, "bf16", "bf16", 1.0, 0.02, 0.02, seed=1001),
    # Prefill with the same shape.
    "c2": LayerSpec("c2", 4096, 2048, 768, 128, 8, 1, 768, "bf16", "bf16", 1.0, 0.02, 0.02, seed=1002),
    "c2_skew": LayerSpec("c2_skew", 4096, 2048, 768, 128, 8, 1, 768, "bf16", "bf16", 1.0, 0.02, 0.02,
                         bias="zipf", seed=1002),
    # DeepSeek-V4-Flash-like: 256 routed top-6, MXFP4 expert weights.
    "c3": LayerSpec("c3", 1, 4096, 2048, 256, 6, 0, 0, "bf16", "mxfp4", 1.0, 0.0, 0.02, seed=1003),
    # 43-layer stack of c3's layer.
    "c4": LayerSpec("c4", 1, 4096, 2048, 256, 6, 0, 0, "bf16", "mxfp4", 1.0, 0.0, 0.02, seed=1004, n_layers=43),
    # c3's layer with NVFP4 expert weights (E2M1 + one E4M3 scale per 16 + an fp32 tensor scale).
    "c3nv": LayerSpec("c3nv", 1, 4096, 2048, 256, 6, 0, 0, "bf16", "nvfp4", 1.0, 0.0, 0.02, scale_lo=0x20,
                      scale_hi=0x3F, seed=1005),
}


def spec(name: str, T: Optional[int] = None) -> LayerSpec:
    s = CONFIGS[name]
    return s if T is None else s.with_T(T)


# ----------------------------------------------------------------------------------------------
# Host generation (numpy)
# ----------------------------------------------------------------------------------------------
def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def host_normal(n: int, key: int, sigma: float, dtype: str, start: int = 0) -> np.ndarray:
    lib = _load_host()
    if dtype == "f32":
        out = np.empty(n, np.float32)
        lib.mg_fill_normal_f32(_ptr(out), n, key, normal_scale(sigma), start)
    elif dtype == "bf16":
        out = np.empty(n, np.uint16)
        lib.mg_fill_normal_bf16(_ptr(out), n, key, normal_scale(sigma), start)
    else:
        raise ValueError(dtype)
    return out


def x_row_sub(t: int, attempt: int) -> int:
    return ((int(attempt) & 0xFFFFFFFF) << 32) | (int(t) & 0xFFFFFFFF)


def host_x(s: LayerSpec, layer: int = 0, attempts: Optional[np.ndarray] = None,
           rows: Optional[Sequence[int]] = None, sigma: Optional[float] = None) -> np.ndarray:
    """Activations x [len(rows), d] (float32 or bf16 bits as uint16)."""
    rows = range(s.T) if rows is None else rows
    kx = tensor_key(s.seed, layer, TAG_X)
    sig = s.sigma_x if sigma is None else sigma
    out = []
    for t in rows:
        a = 0 if attempts is None else int(attempts[t])
        out.append(host_normal(s.d, derive(kx, x_row_sub(t, a)), sig, s.act))
    if not out:
        return np.zeros((0, s.d), np.float32 if s.act == "f32" else np.uint16)
    return np.stack(out)


def host_h0(s: LayerSpec) -> np.ndarray:
    """fp32 residual stream entering the first layer of a stack, [T, d]."""
    kh = tensor_key(s.seed, 0, TAG_H0)
    return np.stack([host_normal(s.d, derive(kh, t), 1.0, "f32") for t in range(s.T)])


def host_router(s: LayerSpec, layer: int = 0):
    """(W_r [E, d] in the activation dtype, b [E] float32)."""
    wr = host_normal(s.E * s.d, tensor_key(s.seed, layer, TAG_WR), s.sigma_r, s.act).reshape(s.E, s.d)
    return wr, router_bias(s, layer)


def router_bias(s: LayerSpec, layer: int = 0) -> np.ndarray:
    """Zero, or the skewed prior b_e = -1.1 ln(r_e), r a seeded permutation of 1..E, so that the
    routing odds before the token's own logit follow a Zipf(1.1) law over experts."""
    if s.bias == "zero":
        return np.zeros(s.E, np.float32)
    kp = tensor_key(s.seed, layer, TAG_PERM)
    r = list(range(1, s.E + 1))
    for i in range(s.E - 1, 0, -1):  # Fisher-Yates with the seeded stream
        j = ((word(kp, i) >> 32) * (i + 1)) >> 32
        r[i], r[j] = r[j], r[i]
    return np.array([-1.1 * math.log(v) for v in r], np.float32)


# NVFP4 tensor scales (fp32, one per weight tensor) of the synthetic layers: gate/up, down.
NVFP4_GSCALE = (0.3, 0.6)
# NVFP4 block-scale bytes are drawn uniformly over E4M3 codes 0x20..0x3F: 2^-3 .. 1.875.
NVFP4_SCALE_LO, NVFP4_SCALE_HI = 0x20, 0x3F


def host_experts(s: LayerSpec, layer: int = 0, experts: Optional[Sequence[int]] = None, shared: bool = False):
    """Expert weights for the listed experts (all when None), stacked in that order.

    Returns dict with w13 [n, 2f, d], w2 [n, d, f] (float32 / bf16 bits / MXFP4 code bytes
    [n, 2f, d/2] and [n, d, f/2]) and for MXFP4 w13_scale [n, 2f, d/32], w2_scale [n, d, f/32].
    With shared=True it returns the shared expert's tensors (n = 1, f = f_shared).
    """
    lib = _load_host()
    if shared:
        experts = [0]
        f = s.f_shared
        tags = (TAG_S13, TAG_S2, TAG_S13S, TAG_S2S)
    else:
        experts = list(range(s.E)) if experts is None else list(experts)
        f = s.f
        tags = (TAG_W13, TAG_W2, TAG_W13S, TAG_W2S)
    n = len(experts)
    d = s.d
    k13, k2, k13s, k2s = (tensor_key(s.seed, layer, t) for t in tags)
    out = {}
    if s.wt in ("f32", "bf16"):
        dt = np.float32 if s.wt == "f32" else np.uint16
        w13 = np.empty((n, 2 * f, d), dt)
        w2 = np.empty((n, d, f), dt)
        c = normal_scale(s.sigma_w)
        fill = lib.mg_fill_normal_f32_experts if s.wt == "f32" else lib.mg_fill_normal_bf16_experts
        for i, e in enumerate(experts):
            fill(_ptr(w13[i]), 2 * f * d, e, 1, k13, c)
            fill(_ptr(w2[i]), d * f, e, 1, k2, c)
        out["w13"], out["w2"] = w13, w2
    elif s.wt == "mxfp4":
        assert d % 32 == 0 and f % 32 == 0
        w13 = np.empty((n, 2 * f, d // 2), np.uint8)
        w2 = np.empty((n, d, f // 2), np.uint8)
        w13s = np.empty((n, 2 * f, d // 32), np.uint8)
        w2s = np.empty((n, d, f // 32), np.uint8)
        for i, e in enumerate(experts):
            lib.mg_fill_bytes_experts(_ptr(w13[i]), w13[i].size, e, 1, k13)
            lib.mg_fill_bytes_experts(_ptr(w2[i]), w2[i].size, e, 1, k2)
            lib.mg_fill_scale_bytes_experts(_ptr(w13s[i]), w13s[i].size, e, 1, k13s, s.scale_lo, s.scale_hi)
            lib.mg_fill_scale_bytes_experts(_ptr(w2s[i]), w2s[i].size, e, 1, k2s, s.scale_lo, s.scale_hi)
        out.update(w13=w13, w2=w2, w13_scale=w13s, w2_scale=w2s)
    elif s.wt == "nvfp4":
        assert d % 32 == 0 and f % 32 == 0
        w13 = np.empty((n, 2 * f, d // 2), np.uint8)
        w2 = np.empty((n, d, f // 2), np.uint8)
        w13s = np.empty((n, 2 * f, d // 16), np.uint8)
        w2s = np.empty((n, d, f // 16), np.uint8)
        for i, e in enumerate(experts):
            lib.mg_fill_bytes_experts(_ptr(w13[i]), w13[i].size, e, 1, k13)
            lib.mg_fill_bytes_experts(_ptr(w2[i]), w2[i].size, e, 1, k2)
            lib.mg_fill_scale_bytes_experts(_ptr(w13s[i]), w13s[i].size, e, 1, k13s, s.scale_lo, s.scale_hi)
            lib.mg_fill_scale_bytes_experts(_ptr(w2s[i]), w2s[i].size, e, 1, k2s, s.scale_lo, s.scale_hi)
        out.update(w13=w13, w2=w2, w13_scale=w13s, w2_scale=w2s, w13_gscale=NVFP4_GSCALE[0],
                   w2_gscale=NVFP4_GSCALE[1])
    else:
        raise ValueError(s.wt)
    return out


# ----------------------------------------------------------------------------------------------
# Device generation (torch tensors on the GPU; torch is plumbing here)
# ----------------------------------------------------------------------------------------------
def _stream_handle():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(rc):
    if rc != 0:
        raise RuntimeError(f"device generator failed with HIP error {rc}")


def device_experts(s: LayerSpec, layer: int = 0, shared: bool = False, device="cuda"):
    """The same tensors as host_experts(s, layer) for all experts, generated in device memory."""
    import torch
    lib = _load_dev()
    st = _stream_handle()
    if shared:
        n, f = 1, s.f_shared
        tags = (TAG_S13, TAG_S2, TAG_S13S, TAG_S2S)
    else:
        n, f = s.E, s.f
        tags = (TAG_W13, TAG_W2, TAG_W13S, TAG_W2S)
    d = s.d
    k13, k2, k13s, k2s = (tensor_key(s.seed, layer, t) for t in tags)
    out = {}
    if s.wt in ("f32", "bf16"):
        tdt = torch.float32 if s.wt == "f32" else torch.bfloat16
        w13 = torch.empty((n, 2 * f, d), dtype=tdt, device=device)
        w2 = torch.empty((n, d, f), dtype=tdt, device=device)
        c = normal_scale(s.sigma_w)
        fill = lib.mgd_fill_normal_f32 if s.wt == "f32" else lib.mgd_fill_normal_bf16
        _check(fill(w13.data_ptr(), 2 * f * d, 0, n, k13, c, 1, st))
        _check(fill(w2.data_ptr(), d * f, 0, n, k2, c, 1, st))
        out["w13"], out["w2"] = w13, w2
    else:
        blk = 16 if s.wt == "nvfp4" else 32  # elements per scale byte
        w13 = torch.empty((n, 2 * f, d // 2), dtype=torch.uint8, device=device)
        w2 = torch.empty((n, d, f // 2), dtype=torch.uint8, device=device)
        w13s = torch.empty((n, 2 * f, d // blk), dtype=torch.uint8, device=device)
        w2s = torch.empty((n, d, f // blk), dtype=torch.uint8, device=device)
        _check(lib.mgd_fill_bytes(w13.data_ptr(), w13[0].numel(), 0, n, k13, 1, st))
        _check(lib.mgd_fill_bytes(w2.data_ptr(), w2[0].numel(), 0, n, k2, 1, st))
        _check(lib.mgd_fill_scale_bytes(w13s.data_ptr(), w13s[0].numel(), 0, n, k13s, s.scale_lo, s.scale_hi, 1, st))
        _check(lib.mgd_fill_scale_bytes(w2s.data_ptr(), w2s[0].numel(), 0, n, k2s, s.scale_lo, s.scale_hi, 1, st))
        out.update(w13=w13, w2=w2, w13_scale=w13s, w2_scale=w2s)
        if s.wt == "nvfp4":
            out.update(w13_gscale=NVFP4_GSCALE[0], w2_gscale=NVFP4_GSCALE[1])
    return out


def to_device(a: np.ndarray, act: str, device="cuda"):
    """Copy a host array to the device, reinterpreting uint16 bf16 bits as torch.bfloat16."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if act == "bf16" and a.dtype == np.uint16:
        t = t.view(torch.int16).view(torch.bfloat16) if hasattr(torch, "uint16") is False else t.view(torch.bfloat16)
    return t.to(device)


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint32) << 16).view(np.float32)
