"""The C-ABI library without a GPU: it loads, exports every entry point include/moe.h
declares, and rejects invalid arguments on the host before any launch (no device is
touched: every call below must return its status without reaching HIP)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import sparse_mixture_experts_16_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    txt = open(os.path.join(ROOT, "include", "moe.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", txt)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert set(names) == set(moe.EXPORTS), names
    lib = ctypes.CDLL(moe.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def _shape(**kw):
    base = dict(T=4, d_model=256, d_ff=128, n_experts=8, top_k=2, n_shared=0, shared_d_ff=0,
                act_dtype=moe.MOE_BF16, weight_dtype=moe.MOE_BF16, flags=0)
    base.update(kw)
    return moe.Shape(**base)


FAKE = 0x10000  # 16-byte aligned non-null address: never dereferenced because validation fails first


def _layer(shape, x=FAKE, wr=FAKE, out=FAKE, w=None, ws=FAKE, ws_bytes=1 << 40):
    W = w or moe.Weights(w13=FAKE, w2=FAKE)
    return moe.lib().moe_layer_forward(ctypes.byref(shape), x, wr, None, ctypes.byref(W), out, None, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(top_k=0), moe.MOE_ERR_INVALID_ARG),
    (dict(top_k=9), moe.MOE_ERR_INVALID_ARG),
    (dict(T=-1), moe.MOE_ERR_INVALID_ARG),
    (dict(d_model=0), moe.MOE_ERR_INVALID_ARG),
    (dict(n_shared=2), moe.MOE_ERR_INVALID_ARG),
    (dict(n_shared=1, shared_d_ff=0), moe.MOE_ERR_INVALID_ARG),
    (dict(act_dtype=moe.MOE_F32, weight_dtype=moe.MOE_BF16), moe.MOE_ERR_UNSUPPORTED),
    (dict(act_dtype=moe.MOE_F32, weight_dtype=moe.MOE_MXFP4), moe.MOE_ERR_UNSUPPORTED),
    (dict(act_dtype=moe.MOE_F32, weight_dtype=moe.MOE_NVFP4), moe.MOE_ERR_UNSUPPORTED),
    (dict(act_dtype=moe.MOE_NVFP4), moe.MOE_ERR_INVALID_ARG),
    (dict(act_dtype=moe.MOE_MXFP4), moe.MOE_ERR_INVALID_ARG),
    (dict(weight_dtype=7), moe.MOE_ERR_INVALID_ARG),
    (dict(n_experts=2048, top_k=2), moe.MOE_ERR_UNSUPPORTED),
    (dict(n_experts=128, top_k=65), moe.MOE_ERR_UNSUPPORTED),
    (dict(weight_dtype=moe.MOE_MXFP4, d_model=48), moe.MOE_ERR_INVALID_ARG),
    (dict(weight_dtype=moe.MOE_MXFP4, d_ff=80), moe.MOE_ERR_INVALID_ARG),
    (dict(weight_dtype=moe.MOE_NVFP4, d_model=48), moe.MOE_ERR_INVALID_ARG),
    (dict(weight_dtype=moe.MOE_NVFP4, n_shared=1, shared_d_ff=80), moe.MOE_ERR_INVALID_ARG),
    (dict(d_model=100), moe.MOE_ERR_INVALID_ARG),
    (dict(flags=1 << 20), moe.MOE_ERR_INVALID_ARG),
    (dict(flags=moe.F_MX_GEMM), moe.MOE_ERR_UNSUPPORTED),                    # MX GEMM needs MXFP4 weights
    (dict(weight_dtype=moe.MOE_NVFP4, flags=moe.F_MX_GEMM), moe.MOE_ERR_UNSUPPORTED),
    (dict(flags=moe.F_FORCE_GEMV | moe.F_FORCE_GEMM), moe.MOE_ERR_INVALID_ARG),
])
def test_invalid_shapes_rejected(kw, status):
    s = _shape(**kw)
    assert _layer(s) == status
    assert moe.workspace_size(s) == 0


def test_null_and_misaligned_pointers_rejected():
    s = _shape()
    assert _layer(s, x=None) == moe.MOE_ERR_INVALID_ARG
    assert _layer(s, wr=None) == moe.MOE_ERR_INVALID_ARG
    assert _layer(s, out=FAKE + 4) == moe.MOE_ERR_INVALID_ARG
    assert _layer(s, w=moe.Weights(w13=FAKE, w2=None)) == moe.MOE_ERR_INVALID_ARG
    # MXFP4 needs its scale arrays
    s4 = _shape(weight_dtype=moe.MOE_MXFP4)
    assert _layer(s4, w=moe.Weights(w13=FAKE, w2=FAKE)) == moe.MOE_ERR_INVALID_ARG
    # and so does NVFP4 (a tensor scale alone is not enough)
    s5 = _shape(weight_dtype=moe.MOE_NVFP4)
    assert _layer(s5, w=moe.Weights(w13=FAKE, w2=FAKE, w13_gscale=1.0, w2_gscale=1.0)) == moe.MOE_ERR_INVALID_ARG
    assert _layer(s5, w=moe.Weights(w13=FAKE, w2=FAKE, w13_scale=FAKE)) == moe.MOE_ERR_INVALID_ARG
    # a shared expert needs its weights
    s1 = _shape(n_shared=1, shared_d_ff=64)
    assert _layer(s1) == moe.MOE_ERR_INVALID_ARG


def test_workspace_too_small_rejected():
    s = _shape()
    need = moe.workspace_size(s)
    assert need > 0
    assert _layer(s, ws_bytes=need - 1) == moe.MOE_ERR_WORKSPACE
    assert _layer(s, ws=None) == moe.MOE_ERR_WORKSPACE


def test_empty_batch_is_ok_without_launch():
    s = _shape(T=0)
    assert _layer(s, x=None, wr=None, out=None, ws=None, ws_bytes=0) == moe.MOE_OK


def test_other_entry_points_validate():
    L = moe.lib()
    s = _shape(top_k=0)
    assert L.moe_route(ctypes.byref(s), FAKE, FAKE, None, None, FAKE, FAKE, None, FAKE, 1 << 30, None) == moe.MOE_ERR_INVALID_ARG
    s = _shape()
    assert L.moe_route(ctypes.byref(s), None, FAKE, None, None, FAKE, FAKE, None, FAKE, 1 << 30, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_permute(ctypes.byref(s), FAKE, FAKE, FAKE, None, FAKE, FAKE, 1 << 30, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_permute(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None) == moe.MOE_ERR_WORKSPACE
    W = moe.Weights(w13=FAKE, w2=FAKE)
    assert L.moe_grouped_ffn(ctypes.byref(s), FAKE, FAKE, FAKE, ctypes.byref(W), None, None, FAKE, 1 << 30, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_combine(ctypes.byref(s), FAKE, None, FAKE, None, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_mxfp4_dequant(FAKE, FAKE, 4, 48, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_mxfp4_dequant(FAKE, FAKE, -1, 64, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_mxfp4_dequant(FAKE, FAKE, 0, 64, FAKE, None) == moe.MOE_OK
    assert L.moe_nvfp4_dequant(FAKE, FAKE, 1.0, 4, 48, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_nvfp4_dequant(FAKE, FAKE, 1.0, -1, 64, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_nvfp4_dequant(FAKE, FAKE + 1, 1.0, 4, 64, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_nvfp4_dequant(FAKE, None, 1.0, 4, 64, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_nvfp4_dequant(FAKE, FAKE, 1.0, 0, 64, FAKE, None) == moe.MOE_OK
    assert L.moe_mxfp8_quantize(FAKE, moe.MOE_BF16, 4, 48, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_mxfp8_quantize(FAKE, moe.MOE_MXFP4, 4, 64, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_mxfp8_quantize(FAKE + 4, moe.MOE_F32, 4, 64, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_mxfp8_quantize(FAKE, moe.MOE_F32, 0, 64, FAKE, FAKE, None) == moe.MOE_OK
    # the MX stages: MXFP4 weights and 128-multiple sizes only; argument checks before any launch
    mx = _shape(weight_dtype=moe.MOE_MXFP4, d_model=256, d_ff=128)
    W4 = moe.Weights(w13=FAKE, w2=FAKE, w13_scale=FAKE, w2_scale=FAKE)
    assert L.moe_mx_gate_up(ctypes.byref(_shape()), FAKE, FAKE, FAKE, ctypes.byref(W4), FAKE, FAKE, FAKE, 1 << 40,
                            None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_mx_gate_up(ctypes.byref(_shape(weight_dtype=moe.MOE_MXFP4, d_model=96 * 2, d_ff=128)), FAKE, FAKE,
                            FAKE, ctypes.byref(W4), FAKE, FAKE, FAKE, 1 << 40, None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_mx_gate_up(ctypes.byref(mx), FAKE, FAKE, FAKE, ctypes.byref(W4), None, FAKE, FAKE, 1 << 40,
                            None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_mx_gate_up(ctypes.byref(mx), FAKE, FAKE, FAKE, ctypes.byref(W4), FAKE, FAKE, FAKE, 1,
                            None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_mx_down(ctypes.byref(mx), FAKE, FAKE, FAKE, ctypes.byref(W4), None, None, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_mx_down(ctypes.byref(_shape(weight_dtype=moe.MOE_MXFP4, d_model=256, d_ff=128, T=0)), None, None,
                         None, ctypes.byref(W4), None, None, None) == moe.MOE_OK
    arr = (ctypes.c_void_p * 1)(FAKE)
    assert L.moe_stack_forward(ctypes.byref(s), -1, FAKE, arr, None, ctypes.byref(W), None, FAKE, 1 << 30,
                               None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_stack_forward(ctypes.byref(s), 1, FAKE + 8, arr, None, ctypes.byref(W), None, FAKE, 1 << 30,
                               None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_stack_forward(ctypes.byref(s), 1, FAKE, arr, None, ctypes.byref(W), FAKE + 4, FAKE, 1 << 30,
                               None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_stack_forward(ctypes.byref(s), 1, FAKE, arr, None, ctypes.byref(W), None, FAKE, 1,
                               None) == moe.MOE_ERR_WORKSPACE
    # the partial layer needs its expert mask, 16-byte aligned, and validates like the full layer
    masked = lambda s_, m, out=FAKE: L.moe_layer_forward_masked(ctypes.byref(s_), FAKE, FAKE, None, ctypes.byref(W), m,
                                                               out, None, FAKE, 1 << 40, None)
    assert masked(s, None) == moe.MOE_ERR_INVALID_ARG
    assert masked(s, FAKE + 1) == moe.MOE_ERR_INVALID_ARG
    assert masked(s, FAKE, out=None) == moe.MOE_ERR_INVALID_ARG
    assert masked(_shape(top_k=0), FAKE) == moe.MOE_ERR_INVALID_ARG
    assert masked(_shape(T=0), FAKE) == moe.MOE_OK


def test_noalloc_validates_before_any_device_call():
    L = moe.lib()
    W = moe.Weights(w13=FAKE, w2=FAKE)
    call = lambda s_, x=FAKE, out=FAKE: L.moe_layer_forward_noalloc(ctypes.byref(s_), x, FAKE, None, ctypes.byref(W),
                                                                    out, None, None)
    assert call(_shape(top_k=0)) == moe.MOE_ERR_INVALID_ARG
    assert call(_shape(), x=None) == moe.MOE_ERR_INVALID_ARG
    assert call(_shape(), out=FAKE + 2) == moe.MOE_ERR_INVALID_ARG
    assert call(_shape(T=0), x=None, out=None) == moe.MOE_OK
    big = _shape(T=4096, d_model=2048, d_ff=768, n_experts=128, top_k=8)
    assert moe.workspace_size(big) > moe.NOALLOC_SCRATCH_BYTES
    assert call(big) == moe.MOE_ERR_SCRATCH_LIMIT


def test_status_strings():
    for st in (0, -1, -2, -3, -4, -5, 5):
        assert isinstance(moe.lib().moe_status_string(st), bytes)


def test_stack_persistent_validation_on_host():
    """The persistent stack takes one token, bf16 activations, MXFP4 weights, no shared expert and
    the single-pass decode shapes; everything else is refused before any launch."""
    L = moe.lib()
    ok = _shape(T=1, d_model=512, d_ff=256, n_experts=16, top_k=4, weight_dtype=moe.MOE_MXFP4)
    W4 = moe.Weights(w13=FAKE, w2=FAKE, w13_scale=FAKE, w2_scale=FAKE)
    arr = (ctypes.c_void_p * 2)(FAKE, FAKE)
    Ws = (moe.Weights * 2)(W4, W4)
    size = L.moe_stack_persistent_workspace_size
    assert size(ctypes.byref(ok), 2) > 0
    # the barrier words plus, per layer, logits, x, a and (between layers) h, each 256-byte aligned
    up = lambda v: (v + 255) // 256 * 256
    per = up(16 * 4) + up(512 * 2) + up(4 * 256 * 4)
    assert size(ctypes.byref(ok), 2) == up(size(ctypes.byref(ok), 1) + per + up(512 // 8 * 128))
    assert size(ctypes.byref(ok), 100) == size(ctypes.byref(ok), 48)  # 48 layers per launch, regions reused
    for bad in (dict(T=2), dict(weight_dtype=moe.MOE_BF16), dict(weight_dtype=moe.MOE_NVFP4),
                dict(n_shared=1, shared_d_ff=256), dict(d_model=4096 + 32), dict(d_ff=2048 + 32),
                dict(flags=moe.F_FORCE_GEMM)):
        s = _shape(**{**dict(T=1, d_model=512, d_ff=256, n_experts=16, top_k=4, weight_dtype=moe.MOE_MXFP4), **bad})
        assert size(ctypes.byref(s), 2) == 0, bad
        assert L.moe_stack_forward_persistent(ctypes.byref(s), 2, FAKE, arr, None, Ws, None, FAKE, 1 << 40,
                                              None) == moe.MOE_ERR_UNSUPPORTED, bad
    call = lambda n=2, h=FAKE, idx=None, ws=FAKE, nb=1 << 40, wr=arr: L.moe_stack_forward_persistent(
        ctypes.byref(ok), n, h, wr, None, Ws, idx, ws, nb, None)
    assert call(n=-1) == moe.MOE_ERR_INVALID_ARG
    assert call(n=0) == moe.MOE_OK
    assert call(h=FAKE + 8) == moe.MOE_ERR_INVALID_ARG
    assert call(idx=FAKE + 4) == moe.MOE_ERR_INVALID_ARG
    assert call(wr=(ctypes.c_void_p * 2)(FAKE, None)) == moe.MOE_ERR_INVALID_ARG
    assert call(ws=None) == moe.MOE_ERR_WORKSPACE
    assert call(nb=size(ctypes.byref(ok), 2) - 1) == moe.MOE_ERR_WORKSPACE
    assert L.moe_stack_persistent_set_spin_limit(-1) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_stack_persistent_status(None, ctypes.byref(ctypes.c_int32()), None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_stack_persistent_status(FAKE + 4, ctypes.byref(ctypes.c_int32()), None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_stack_persistent_status(FAKE, None, None) == moe.MOE_ERR_INVALID_ARG
