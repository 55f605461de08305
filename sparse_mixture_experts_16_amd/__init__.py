"""Python binding of libmoe.so, the gfx950 routed mixture-of-experts layer.

Argument marshalling only: every step of the layer runs in the HIP kernels behind the
C-ABI declared in include/moe.h.  torch provides device memory and the current HIP
stream; tensors are passed as raw device pointers.  There is no CPU fallback: importing
this package fails if libmoe.so is not built, and every call raises on a non-OK status.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

# torch ships its own HIP runtime (soname libamdhip64.so.7).  It must be loaded before
# libmoe.so so that the library's libamdhip64.so.7 dependency binds to that same runtime;
# loading libmoe.so first would bring in a second HIP runtime and torch would then load
# its own copy beside it.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_ERR_SCRATCH_LIMIT = -5
NOALLOC_SCRATCH_BYTES = 64 << 20
MOE_F32, MOE_BF16, MOE_MXFP4, MOE_NVFP4 = 0, 1, 2, 3
F_NO_RENORM, F_ACCUMULATE, F_FORCE_GEMV, F_FORCE_GEMM, F_MX_GEMM = 1 << 0, 1 << 1, 1 << 3, 1 << 4, 1 << 5
MAX_EXPERTS, MAX_TOPK = 1024, 64
_DT = {"f32": MOE_F32, "bf16": MOE_BF16, "mxfp4": MOE_MXFP4, "nvfp4": MOE_NVFP4}

EXPORTS = ["moe_workspace_size", "moe_status_string", "moe_route", "moe_permute", "moe_grouped_ffn",
           "moe_combine", "moe_layer_forward", "moe_layer_forward_noalloc", "moe_layer_forward_masked",
           "moe_stack_forward", "moe_stack_persistent_workspace_size", "moe_stack_forward_persistent",
           "moe_stack_persistent_status", "moe_stack_persistent_set_spin_limit", "moe_mxfp4_dequant",
           "moe_nvfp4_dequant", "moe_mxfp8_quantize", "moe_mx_gate_up", "moe_mx_down",
           "moe_profile_kernel"]
KERNEL_FFN_UP, KERNEL_FFN_DOWN = 0, 1


class Shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("shared_d_ff", ctypes.c_int32), ("act_dtype", ctypes.c_int32), ("weight_dtype", ctypes.c_int32),
                ("flags", ctypes.c_uint32)]


class Weights(ctypes.Structure):
    _fields_ = ([(n, ctypes.c_void_p) for n in ("w13", "w2", "w13_scale", "w2_scale", "s13", "s2", "s13_scale", "s2_scale")]
                + [(n, ctypes.c_float) for n in ("w13_gscale", "w2_gscale", "s13_gscale", "s2_gscale")])


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build the HIP library first (__graft_entry__.build())")
_lib = ctypes.CDLL(LIB_PATH)
_vp, _sz, _i32, _i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
_SP, _WP = ctypes.POINTER(Shape), ctypes.POINTER(Weights)
_lib.moe_workspace_size.restype = _sz
_lib.moe_workspace_size.argtypes = [_SP]
_lib.moe_status_string.restype = ctypes.c_char_p
_lib.moe_status_string.argtypes = [ctypes.c_int]
_lib.moe_route.argtypes = [_SP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.moe_permute.argtypes = [_SP, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.moe_grouped_ffn.argtypes = [_SP, _vp, _vp, _vp, _WP, _vp, _vp, _vp, _sz, _vp]
_lib.moe_combine.argtypes = [_SP, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.moe_layer_forward.argtypes = [_SP, _vp, _vp, _vp, _WP, _vp, _vp, _vp, _sz, _vp]
_lib.moe_layer_forward_noalloc.argtypes = [_SP, _vp, _vp, _vp, _WP, _vp, _vp, _vp]
_lib.moe_layer_forward_masked.argtypes = [_SP, _vp, _vp, _vp, _WP, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.moe_stack_forward.argtypes = [_SP, _i32, _vp, ctypes.POINTER(_vp), ctypes.POINTER(_vp), _WP, _vp, _vp, _sz, _vp]
_lib.moe_stack_persistent_workspace_size.argtypes = [_SP, _i32]
_lib.moe_stack_forward_persistent.argtypes = [_SP, _i32, _vp, ctypes.POINTER(_vp), ctypes.POINTER(_vp), _WP, _vp, _vp,
                                              _sz, _vp]
_lib.moe_stack_persistent_status.argtypes = [_vp, ctypes.POINTER(_i32), _vp]
_lib.moe_stack_persistent_set_spin_limit.argtypes = [_i32]
_lib.moe_mxfp4_dequant.argtypes = [_vp, _vp, _i64, _i64, _vp, _vp]
_lib.moe_nvfp4_dequant.argtypes = [_vp, _vp, ctypes.c_float, _i64, _i64, _vp, _vp]
_lib.moe_mxfp8_quantize.argtypes = [_vp, _i32, _i64, _i64, _vp, _vp, _vp]
_lib.moe_mx_gate_up.argtypes = [_SP, _vp, _vp, _vp, _WP, _vp, _vp, _vp, _sz, _vp]
_lib.moe_mx_down.argtypes = [_SP, _vp, _vp, _vp, _WP, _vp, _vp, _vp]
_lib.moe_profile_kernel.argtypes = [ctypes.c_int, _vp, _vp]
for _n in EXPORTS[2:]:
    getattr(_lib, _n).restype = ctypes.c_int
_lib.moe_stack_persistent_workspace_size.restype = _sz


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_lib.moe_status_string(status).decode()} ({status})")


def lib():
    return _lib


def _check(rc: int, what: str):
    if rc != MOE_OK:
        raise MoeError(rc, what)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def make_shape(spec=None, *, T=None, d=None, f=None, E=None, k=None, n_shared=None, f_shared=None, act=None,
               wt=None, flags: int = 0) -> Shape:
    """Shape from a spec object (attributes T, d, f, E, k, n_shared, f_shared, act, wt) and overrides."""
    g = (lambda n, v: v if v is not None else getattr(spec, n))
    return Shape(T=g("T", T), d_model=g("d", d), d_ff=g("f", f), n_experts=g("E", E), top_k=g("k", k),
                 n_shared=g("n_shared", n_shared), shared_d_ff=g("f_shared", f_shared),
                 act_dtype=_DT[g("act", act)], weight_dtype=_DT[g("wt", wt)], flags=flags)


def workspace_size(shape: Shape) -> int:
    return int(_lib.moe_workspace_size(ctypes.byref(shape)))


_ws_cache = {}


def workspace(shape: Shape, device="cuda"):
    """A device workspace of at least moe_workspace_size(shape) bytes (cached, grown on demand)."""
    import torch
    n = max(workspace_size(shape), 256)
    dev = torch.device(device)
    cur = _ws_cache.get(dev)
    if cur is None or cur.numel() < n:
        cur = torch.empty(n, dtype=torch.uint8, device=dev)  # needs no initialisation
        _ws_cache[dev] = cur
    return cur


def make_weights(w: dict, shared: Optional[dict] = None) -> Weights:
    W = Weights()
    W.w13, W.w2 = _ptr(w["w13"]), _ptr(w["w2"])
    W.w13_scale, W.w2_scale = _ptr(w.get("w13_scale")), _ptr(w.get("w2_scale"))
    W.w13_gscale, W.w2_gscale = float(w.get("w13_gscale", 1.0)), float(w.get("w2_gscale", 1.0))
    W.s13_gscale = W.s2_gscale = 1.0
    if shared is not None:
        W.s13, W.s2 = _ptr(shared["w13"]), _ptr(shared["w2"])
        W.s13_scale, W.s2_scale = _ptr(shared.get("w13_scale")), _ptr(shared.get("w2_scale"))
        W.s13_gscale, W.s2_gscale = float(shared.get("w13_gscale", 1.0)), float(shared.get("w2_gscale", 1.0))
    return W


def _act_torch_dtype(shape: Shape):
    import torch
    return torch.float32 if shape.act_dtype == MOE_F32 else torch.bfloat16


# ------------------------------------------------------------------------------------------------
# Raw entry points (same names as the C-ABI, minus the prefix); all tensors on the device
# ------------------------------------------------------------------------------------------------
def route(shape: Shape, x, w_router, b_router, topk_idx, topk_w, logits_in=None, logits_out=None, ws=None,
          stream=None):
    ws = workspace(shape) if ws is None else ws
    _check(_lib.moe_route(ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(b_router), _ptr(logits_in),
                          _ptr(topk_idx), _ptr(topk_w), _ptr(logits_out), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_route")


def permute(shape: Shape, topk_idx, counts, offsets, perm, inv_perm, ws=None, stream=None):
    ws = workspace(shape) if ws is None else ws
    _check(_lib.moe_permute(ctypes.byref(shape), _ptr(topk_idx), _ptr(counts), _ptr(offsets), _ptr(perm),
                            _ptr(inv_perm), _ptr(ws), ws.numel(), _stream(stream)), "moe_permute")


def grouped_ffn(shape: Shape, x, perm, offsets, weights: Weights, y_sorted, y_shared=None, ws=None, stream=None):
    ws = workspace(shape) if ws is None else ws
    _check(_lib.moe_grouped_ffn(ctypes.byref(shape), _ptr(x), _ptr(perm), _ptr(offsets), ctypes.byref(weights),
                                _ptr(y_sorted), _ptr(y_shared), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_grouped_ffn")


def combine(shape: Shape, y_sorted, inv_perm, topk_w, y_shared, out, stream=None):
    _check(_lib.moe_combine(ctypes.byref(shape), _ptr(y_sorted), _ptr(inv_perm), _ptr(topk_w), _ptr(y_shared),
                            _ptr(out), _stream(stream)), "moe_combine")


def layer_forward_raw(shape: Shape, x, w_router, b_router, weights: Weights, out, topk_idx_out=None, ws=None,
                      stream=None):
    ws = workspace(shape) if ws is None else ws
    _check(_lib.moe_layer_forward(ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(b_router),
                                  ctypes.byref(weights), _ptr(out), _ptr(topk_idx_out), _ptr(ws), ws.numel(),
                                  _stream(stream)), "moe_layer_forward")


def layer_forward_noalloc_raw(shape: Shape, x, w_router, b_router, weights: Weights, out, topk_idx_out=None,
                              stream=None):
    """moe_layer_forward_noalloc: the layer on the library's own per-GPU scratch area."""
    _check(_lib.moe_layer_forward_noalloc(ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(b_router),
                                          ctypes.byref(weights), _ptr(out), _ptr(topk_idx_out), _stream(stream)),
           "moe_layer_forward_noalloc")


def layer_forward_masked_raw(shape: Shape, x, w_router, b_router, weights: Weights, expert_mask, out,
                             topk_idx_out=None, ws=None, stream=None):
    """moe_layer_forward_masked: expert_mask is a device uint8 tensor of E + 1 bytes."""
    ws = workspace(shape) if ws is None else ws
    _check(_lib.moe_layer_forward_masked(ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(b_router),
                                         ctypes.byref(weights), _ptr(expert_mask), _ptr(out), _ptr(topk_idx_out),
                                         _ptr(ws), ws.numel(), _stream(stream)), "moe_layer_forward_masked")


def stack_forward(shape: Shape, h, w_routers, b_routers, weights_list, ws=None, stream=None, topk_idx_out=None):
    """moe_stack_forward; topk_idx_out (optional) is a device int32 tensor [n_layers, T, k]."""
    n = len(weights_list)
    ws = workspace(shape) if ws is None else ws
    wr = (_vp * n)(*[_ptr(t) for t in w_routers])
    br = (_vp * n)(*[_ptr(t) for t in b_routers]) if b_routers is not None else None
    W = (Weights * n)(*weights_list)
    _check(_lib.moe_stack_forward(ctypes.byref(shape), n, _ptr(h), wr, br, W, _ptr(topk_idx_out), _ptr(ws),
                                  ws.numel(), _stream(stream)), "moe_stack_forward")


def stack_persistent_workspace_size(shape: Shape, n_layers: int) -> int:
    """Bytes of workspace moe_stack_forward_persistent needs (0: shape not supported)."""
    return int(_lib.moe_stack_persistent_workspace_size(ctypes.byref(shape), n_layers))


def stack_forward_persistent(shape: Shape, h, w_routers, b_routers, weights_list, ws, stream=None, topk_idx_out=None):
    """moe_stack_forward_persistent (one token, the whole stack in one cooperative launch per 48 layers);
    ws: a device uint8 tensor of at least stack_persistent_workspace_size bytes."""
    n = len(weights_list)
    wr = (_vp * n)(*[_ptr(t) for t in w_routers])
    br = (_vp * n)(*[_ptr(t) for t in b_routers]) if b_routers is not None else None
    W = (Weights * n)(*weights_list)
    _check(_lib.moe_stack_forward_persistent(ctypes.byref(shape), n, _ptr(h), wr, br, W, _ptr(topk_idx_out),
                                             _ptr(ws), ws.numel(), _stream(stream)), "moe_stack_forward_persistent")


def stack_persistent_status(ws, stream=None) -> int:
    """Synchronises the stream; 0, or 1 if a grid-barrier wait of the last call ran out."""
    v = _i32(0)
    _check(_lib.moe_stack_persistent_status(_ptr(ws), ctypes.byref(v), _stream(stream)), "moe_stack_persistent_status")
    return int(v.value)


def stack_persistent_set_spin_limit(spins: int):
    """Polls of a grid-barrier wait before it gives up (default 1 << 20)."""
    _check(_lib.moe_stack_persistent_set_spin_limit(spins), "moe_stack_persistent_set_spin_limit")


def mxfp4_dequant(codes, scales, out, stream=None):
    rows, half_k = codes.shape[-2] if codes.dim() > 1 else 1, codes.shape[-1]
    rows = codes.numel() // half_k
    _check(_lib.moe_mxfp4_dequant(_ptr(codes), _ptr(scales), rows, 2 * half_k, _ptr(out), _stream(stream)),
           "moe_mxfp4_dequant")


def mxfp8_quantize(x, codes, scales, stream=None):
    """x [rows, K] float32 or bfloat16 -> codes uint8 [rows, K], scales uint8 [rows, K/32]."""
    import torch
    dt = MOE_F32 if x.dtype == torch.float32 else MOE_BF16
    K = x.shape[-1]
    _check(_lib.moe_mxfp8_quantize(_ptr(x), dt, x.numel() // K, K, _ptr(codes), _ptr(scales), _stream(stream)),
           "moe_mxfp8_quantize")


def mx_gate_up(shape: Shape, x, perm, offsets, weights: Weights, a_codes, a_scales, ws=None, stream=None):
    ws = workspace(shape, x.device) if ws is None else ws
    _check(_lib.moe_mx_gate_up(ctypes.byref(shape), _ptr(x), _ptr(perm), _ptr(offsets), ctypes.byref(weights),
                               _ptr(a_codes), _ptr(a_scales), _ptr(ws), ws.numel(), _stream(stream)), "moe_mx_gate_up")


def mx_down(shape: Shape, a_codes, a_scales, offsets, weights: Weights, y_sorted, y_shared=None, stream=None):
    _check(_lib.moe_mx_down(ctypes.byref(shape), _ptr(a_codes), _ptr(a_scales), _ptr(offsets), ctypes.byref(weights),
                            _ptr(y_sorted), _ptr(y_shared), _stream(stream)), "moe_mx_down")


def nvfp4_dequant(codes, scales, gscale, out, stream=None):
    half_k = codes.shape[-1]
    rows = codes.numel() // half_k
    _check(_lib.moe_nvfp4_dequant(_ptr(codes), _ptr(scales), float(gscale), rows, 2 * half_k, _ptr(out),
                                  _stream(stream)), "moe_nvfp4_dequant")


def profile_kernel(kernel: int, ev_start=None, ev_stop=None):
    """Bracket launches of one kernel class with caller-owned hipEvent_t handles (ints)."""
    _check(_lib.moe_profile_kernel(kernel, ev_start, ev_stop), "moe_profile_kernel")


# ------------------------------------------------------------------------------------------------
# Convenience wrapper: allocate outputs, run the whole layer
# ------------------------------------------------------------------------------------------------
def layer_forward(spec, x, w_router, b_router, w: dict, shared: Optional[dict] = None, flags: int = 0, out=None,
                  T: Optional[int] = None, k: Optional[int] = None):
    """Run moe_layer_forward; returns dict(out [T,d] act dtype, topk_idx [T,k] int32)."""
    import torch
    shape = make_shape(spec, T=x.shape[0] if T is None else T, k=k, flags=flags)
    out = torch.empty((shape.T, shape.d_model), dtype=_act_torch_dtype(shape), device=x.device) if out is None else out
    idx = torch.empty((shape.T, shape.top_k), dtype=torch.int32, device=x.device)
    layer_forward_raw(shape, x, w_router, b_router, make_weights(w, shared), out, idx, workspace(shape, x.device))
    return dict(out=out, topk_idx=idx)
