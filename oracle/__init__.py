"""Python access to the CPU oracle (libmoe_ref.so, built from moe_ref.c with gcc).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's CPU-baseline
leg use it; the GPU product path never imports it.  Functions take numpy arrays
(bf16 tensors as uint16 bit patterns) and return numpy arrays; floating results
are float64 except the router logits (float32, the precision selection is taken in).
`spec` arguments are any object with attributes T, d, f, E, k, n_shared, f_shared,
act ('f32'|'bf16') and wt ('f32'|'bf16'|'mxfp4').
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_REF_LIB lets the mutation test load a deliberately broken build of the oracle.
LIB_PATH = os.environ.get("MOE_REF_LIB") or os.path.join(_HERE, "libmoe_ref.so")

F32, BF16, MXFP4, NVFP4 = 0, 1, 2, 3
NO_RENORM, ACCUMULATE, MX_GEMM = 1, 2, 4
_DT = {"f32": F32, "bf16": BF16, "mxfp4": MXFP4, "nvfp4": NVFP4}


class Shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int64), ("f", ctypes.c_int64), ("E", ctypes.c_int64),
                ("k", ctypes.c_int64), ("n_shared", ctypes.c_int64), ("f_shared", ctypes.c_int64),
                ("act_dtype", ctypes.c_int32), ("wt_dtype", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class Weights(ctypes.Structure):
    _fields_ = ([(n, ctypes.c_void_p) for n in ("w13", "w2", "w13_scale", "w2_scale", "s13", "s2", "s13_scale", "s2_scale")]
                + [(n, ctypes.c_float) for n in ("w13_gscale", "w2_gscale", "s13_gscale", "s2_gscale")])


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, sp = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.POINTER(Shape)
        wp = ctypes.POINTER(Weights)
        L.moe_ref_num_threads.restype = ctypes.c_int
        L.moe_ref_mxfp4_dequant.argtypes = [vp, vp, i64, i64, vp]
        L.moe_ref_e4m3_to_f32.argtypes = [vp, i64, vp]
        L.moe_ref_nvfp4_dequant.argtypes = [vp, vp, ctypes.c_float, i64, i64, vp]
        L.moe_ref_mxfp8_quantize.argtypes = [vp, i64, i64, vp, vp]
        L.moe_ref_mx_dot.argtypes = [vp, vp, vp, vp, i64, vp]
        L.moe_ref_router_logits.argtypes = [sp, vp, vp, vp, vp, vp]
        L.moe_ref_topk.argtypes = [sp, vp, vp, vp]
        L.moe_ref_permute.argtypes = [sp, vp, vp, vp, vp, vp]
        L.moe_ref_grouped_ffn.argtypes = [sp, vp, vp, vp, wp, vp, vp]
        L.moe_ref_swiglu_act.argtypes = [sp, vp, vp, vp, wp, vp, vp]
        L.moe_ref_combine.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.moe_ref_layer_forward.argtypes = [sp, vp, vp, vp, wp, vp, vp, vp, vp, vp]
        L.moe_ref_rmsnorm.argtypes = [i64, i64, vp, ctypes.c_double, i32, vp]
        L.moe_ref_stack_layer.argtypes = [sp, vp, vp, vp, wp, vp]
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "oracle needs C-contiguous numpy arrays"
    return a.ctypes.data


def _rc(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def shape(spec, T: Optional[int] = None, flags: int = 0, k: Optional[int] = None, E: Optional[int] = None) -> Shape:
    return Shape(T=spec.T if T is None else T, d=spec.d, f=spec.f, E=spec.E if E is None else E,
                 k=spec.k if k is None else k, n_shared=spec.n_shared, f_shared=spec.f_shared,
                 act_dtype=_DT[spec.act], wt_dtype=_DT[spec.wt], flags=flags)


def weights(w: dict, shared: Optional[dict] = None) -> Weights:
    W = Weights()
    W.w13, W.w2 = _p(w["w13"]), _p(w["w2"])
    W.w13_scale, W.w2_scale = _p(w.get("w13_scale")), _p(w.get("w2_scale"))
    W.w13_gscale, W.w2_gscale = float(w.get("w13_gscale", 1.0)), float(w.get("w2_gscale", 1.0))
    if shared is not None:
        W.s13, W.s2 = _p(shared["w13"]), _p(shared["w2"])
        W.s13_scale, W.s2_scale = _p(shared.get("w13_scale")), _p(shared.get("w2_scale"))
        W.s13_gscale, W.s2_gscale = float(shared.get("w13_gscale", 1.0)), float(shared.get("w2_gscale", 1.0))
    return W


def num_threads() -> int:
    return int(lib().moe_ref_num_threads())


def e4m3_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, np.uint8)
    out = np.empty(b.shape, np.float32)
    _rc(lib().moe_ref_e4m3_to_f32(_p(b), b.size, _p(out)), "e4m3_to_f32")
    return out


def nvfp4_dequant(codes: np.ndarray, scales: np.ndarray, gscale: float) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    rows, half_k = codes.shape[0], codes.shape[1]
    K = 2 * half_k
    out = np.empty((rows, K), np.float32)
    _rc(lib().moe_ref_nvfp4_dequant(_p(codes), _p(scales), ctypes.c_float(gscale), rows, K, _p(out)), "nvfp4_dequant")
    return out


def mxfp8_quantize(v: np.ndarray):
    """fp32 [rows, K] -> (E4M3 codes uint8 [rows, K], E8M0 scales uint8 [rows, K/32])."""
    v = np.ascontiguousarray(v, np.float32)
    rows, K = v.shape
    codes = np.empty((rows, K), np.uint8)
    scales = np.empty((rows, K // 32), np.uint8)
    _rc(lib().moe_ref_mxfp8_quantize(_p(v), rows, K, _p(codes), _p(scales)), "mxfp8_quantize")
    return codes, scales


def mx_dot(xc: np.ndarray, xs: np.ndarray, wc: np.ndarray, ws: np.ndarray) -> float:
    """The MX path's dot product of one MXFP8 row (E4M3 codes [K], E8M0 scales [K/32]) and one
    MXFP4 row (packed codes [K/2], E8M0 scales [K/32]) as the matrix core sums it."""
    xc, xs = np.ascontiguousarray(xc, np.uint8), np.ascontiguousarray(xs, np.uint8)
    wc, ws = np.ascontiguousarray(wc, np.uint8), np.ascontiguousarray(ws, np.uint8)
    K = xc.size
    assert wc.size * 2 == K and xs.size * 32 == K and ws.size * 32 == K
    out = ctypes.c_double()
    _rc(lib().moe_ref_mx_dot(_p(xc), _p(xs), _p(wc), _p(ws), K, ctypes.addressof(out)), "mx_dot")
    return out.value


def mxfp4_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    rows, half_k = codes.shape[0], codes.shape[1]
    K = 2 * half_k
    out = np.empty((rows, K), np.float32)
    _rc(lib().moe_ref_mxfp4_dequant(_p(codes), _p(scales), rows, K, _p(out)), "mxfp4_dequant")
    return out


def router_logits(spec, x, w_router, b=None):
    S = shape(spec, T=x.shape[0])
    l32 = np.empty((x.shape[0], spec.E), np.float32)
    l64 = np.empty((x.shape[0], spec.E), np.float64)
    _rc(lib().moe_ref_router_logits(ctypes.byref(S), _p(x), _p(w_router), _p(b), _p(l32), _p(l64)), "router_logits")
    return l32, l64


def topk(spec, logits: np.ndarray, flags: int = 0, k: Optional[int] = None):
    T, E = logits.shape
    S = shape(spec, T=T, flags=flags, k=k, E=E)
    idx = np.empty((T, S.k), np.int32)
    w = np.empty((T, S.k), np.float64)
    lg = np.ascontiguousarray(logits, np.float32)
    _rc(lib().moe_ref_topk(ctypes.byref(S), _p(lg), _p(idx), _p(w)), "topk")
    return idx, w


def permute(spec, topk_idx: np.ndarray, E: Optional[int] = None):
    T, k = topk_idx.shape
    S = shape(spec, T=T, k=k, E=E)
    counts = np.empty(S.E, np.int32)
    offsets = np.empty(S.E + 1, np.int32)
    perm = np.empty(T * k, np.int32)
    inv = np.empty(T * k, np.int32)
    ti = np.ascontiguousarray(topk_idx, np.int32)
    _rc(lib().moe_ref_permute(ctypes.byref(S), _p(ti), _p(counts), _p(offsets), _p(perm), _p(inv)), "permute")
    return counts, offsets, perm, inv


def grouped_ffn(spec, x, perm, offsets, w: dict, shared: Optional[dict] = None, k: Optional[int] = None,
                E: Optional[int] = None, flags: int = 0):
    T = x.shape[0]
    S = shape(spec, T=T, k=k, E=E, flags=flags)
    ys = np.empty((T * S.k, spec.d), np.float64)
    ysh = np.empty((T, spec.d), np.float64) if shared is not None else None
    W = weights(w, shared)
    _rc(lib().moe_ref_grouped_ffn(ctypes.byref(S), _p(x), _p(perm), _p(offsets), ctypes.byref(W), _p(ys), _p(ysh)),
        "grouped_ffn")
    return ys, ysh


def swiglu_act(spec, x, perm, offsets, w: dict, shared: Optional[dict] = None, flags: int = 0):
    """The grouped FFN's SwiGLU activations (fp64): a_sorted [T*k, f], a_shared [T, f_shared]."""
    T = x.shape[0]
    S = shape(spec, T=T, flags=flags)
    a = np.empty((T * S.k, spec.f), np.float64)
    ash = np.empty((T, spec.f_shared), np.float64) if shared is not None else None
    W = weights(w, shared)
    _rc(lib().moe_ref_swiglu_act(ctypes.byref(S), _p(x), _p(perm), _p(offsets), ctypes.byref(W), _p(a), _p(ash)),
        "swiglu_act")
    return a, ash


def combine(spec, y_sorted, inv_perm, topk_idx, topk_w, y_shared=None, residual=None, expert_mask=None):
    T, k = topk_idx.shape
    S = shape(spec, T=T, k=k)
    out = np.empty((T, spec.d), np.float64)
    _rc(lib().moe_ref_combine(ctypes.byref(S), _p(y_sorted), _p(inv_perm), _p(topk_idx), _p(topk_w), _p(y_shared),
                              _p(residual), _p(expert_mask), _p(out)), "combine")
    return out


def layer_forward(spec, x, w_router, b, w: dict, shared: Optional[dict] = None, flags: int = 0,
                  expert_mask: Optional[np.ndarray] = None, out_init: Optional[np.ndarray] = None,
                  k: Optional[int] = None):
    """Returns dict(out [T,d] f64, topk_idx [T,k], topk_w [T,k] f64, logits [T,E] f32)."""
    T = x.shape[0]
    S = shape(spec, T=T, flags=flags, k=k)
    if shared is None and spec.n_shared:
        raise ValueError("spec has a shared expert but no shared weights were given")
    out = np.zeros((T, spec.d), np.float64) if out_init is None else np.array(out_init, np.float64, copy=True, order="C")
    idx = np.empty((T, S.k), np.int32)
    g = np.empty((T, S.k), np.float64)
    logits = np.empty((T, spec.E), np.float32)
    W = weights(w, shared)
    _rc(lib().moe_ref_layer_forward(ctypes.byref(S), _p(x), _p(w_router), _p(b), ctypes.byref(W), _p(expert_mask),
                                    _p(out), _p(idx), _p(g), _p(logits)), "layer_forward")
    return dict(out=out, topk_idx=idx, topk_w=g, logits=logits)


def rmsnorm(h: np.ndarray, eps: float = 1e-6, dtype: str = "bf16") -> np.ndarray:
    T, d = h.shape
    out = np.empty((T, d), np.float32 if dtype == "f32" else np.uint16)
    hc = np.ascontiguousarray(h, np.float32)
    _rc(lib().moe_ref_rmsnorm(T, d, _p(hc), eps, _DT[dtype], _p(out)), "rmsnorm")
    return out


def stack_layer(spec, h: np.ndarray, w_router, b, w: dict, k: Optional[int] = None):
    """h <- fp32(h + layer(rmsnorm(h))) in place; returns the layer's topk_idx."""
    assert h.dtype == np.float32 and h.flags["C_CONTIGUOUS"]
    T = h.shape[0]
    S = shape(spec, T=T, k=k)
    idx = np.empty((T, S.k), np.int32)
    W = weights(w)
    _rc(lib().moe_ref_stack_layer(ctypes.byref(S), _p(h), _p(w_router), _p(b), ctypes.byref(W), _p(idx)), "stack_layer")
    return idx
