"""GPU parity of moe_stack_forward_persistent (the residual stack for one token as one cooperative
launch per 48 layers, grid barriers between the steps) against moe_stack_forward (three
launches per layer), which the oracle pins layer by layer (tests/test_gpu_parity.py,
tests/test_gpu_stack.py): the two run the same per-row arithmetic in the same orders, so h after
the stack and every layer's selection must agree bit for bit.  The full 43-layer shape is
compared in tests/test_gpu_stack.py on its generated weights.

Shapes: small stacks whose phases leave lanes and workgroups idle (d_model 320: 40 of 512 x
chunks; d_ff 160: 5 of 64 down chunks), several batches of down units per wavefront (k = 8 > 6),
Zipf router biases and none, 50 layers (two launches: 48 + 2), and a token pool so that the
routing changes between calls.  The time-out path is forced from the host (a spin limit of 0)
and must end the launch normally, report status 1, and leave the next call correct.
"""
from __future__ import annotations

import numpy as np
import pytest

import moe_inputs as mi
from _gpu import dev, host

torch = pytest.importorskip("torch")
moe = pytest.importorskip("sparse_mixture_experts_16_amd")

pytestmark = pytest.mark.gpu

SHAPES = [
    # name, d, f, E, k, layers, bias
    ("d512_E16_k4_L5", 512, 256, 16, 4, 5, "zero"),
    ("d320_f160_E40_k5_L3", 320, 160, 40, 5, 3, "zipf"),
    ("d1024_E256_k8_L4", 1024, 512, 256, 8, 4, "zipf"),
    ("d512_E16_k4_L50", 512, 256, 16, 4, 50, "zero"),
]


def _spec(d, f, E, k, L, bias, seed=2100):
    return mi.LayerSpec("stack_small", 1, d, f, E, k, 0, 0, "bf16", "mxfp4", 1.0, 0.0, 0.02, bias=bias,
                        seed=seed + d + E + L, n_layers=L)


def _weights(s):
    wrs, bs, Ws, keep = [], [], [], []
    for l in range(s.n_layers):
        wr, b = mi.host_router(s, l)
        w = mi.device_experts(s, layer=l)
        wrs.append(dev(wr))
        bs.append(dev(b))
        Ws.append(moe.make_weights(w))
        keep.append(w)
    torch.cuda.synchronize()
    return wrs, bs, Ws, keep


def _pws(shape, L):
    n = moe.stack_persistent_workspace_size(shape, L)
    assert n > 0
    return torch.empty(n, dtype=torch.uint8, device="cuda")


def _both(s, shape, wrs, bs, Ws, pws, h0):
    L = s.n_layers
    h_ref = dev(np.ascontiguousarray(h0))
    i_ref = torch.empty((L, 1, s.k), dtype=torch.int32, device="cuda")
    moe.stack_forward(shape, h_ref, wrs, bs, Ws, moe.workspace(shape), topk_idx_out=i_ref)
    h_p = dev(np.ascontiguousarray(h0))
    i_p = torch.full((L, 1, s.k), -1, dtype=torch.int32, device="cuda")
    moe.stack_forward_persistent(shape, h_p, wrs, bs, Ws, pws, topk_idx_out=i_p)
    status = moe.stack_persistent_status(pws)
    return host(h_ref), host(i_ref), host(h_p), host(i_p), status


@pytest.mark.parametrize("name,d,f,E,k,L,bias", SHAPES, ids=[x[0] for x in SHAPES])
def test_persistent_stack_equals_three_launch_stack(name, d, f, E, k, L, bias):
    s = _spec(d, f, E, k, L, bias)
    print(f"persistent stack {name}: generating {L} layers", flush=True)
    wrs, bs, Ws, keep = _weights(s)
    shape = moe.make_shape(s)
    pws = _pws(shape, L)
    h0s = mi.host_h0(s.with_T(3))
    for t in range(3):
        h_ref, i_ref, h_p, i_p, status = _both(s, shape, wrs, bs, Ws, pws, h0s[t:t + 1])
        assert status == 0
        np.testing.assert_array_equal(i_p, i_ref, err_msg=f"{name} token {t}: selections")
        np.testing.assert_array_equal(h_p, h_ref, err_msg=f"{name} token {t}: h after the stack")
        assert np.isfinite(h_p).all()
        print(f"persistent stack {name} token {t}: bit-equal, first-layer experts {i_p[0, 0].tolist()}", flush=True)
    # no router bias at all (NULL array) takes the same path
    if bias == "zero":
        h_ref = dev(np.ascontiguousarray(h0s[:1]))
        moe.stack_forward(shape, h_ref, wrs, None, Ws, moe.workspace(shape))
        h_p = dev(np.ascontiguousarray(h0s[:1]))
        moe.stack_forward_persistent(shape, h_p, wrs, None, Ws, pws)
        assert moe.stack_persistent_status(pws) == 0
        np.testing.assert_array_equal(host(h_p), host(h_ref))
    del keep, Ws, wrs, bs
    torch.cuda.empty_cache()


def test_persistent_stack_time_out_ends_the_launch():
    s = _spec(512, 256, 16, 4, 3, "zero")
    wrs, bs, Ws, keep = _weights(s)
    shape = moe.make_shape(s)
    pws = _pws(shape, 3)
    h0 = mi.host_h0(s.with_T(1))
    h = dev(np.ascontiguousarray(h0))
    moe.stack_persistent_set_spin_limit(0)
    try:
        moe.stack_forward_persistent(shape, h, wrs, bs, Ws, pws)
        status = moe.stack_persistent_status(pws)
    finally:
        moe.stack_persistent_set_spin_limit(1 << 20)
    print(f"persistent stack with spin limit 0: status {status}", flush=True)
    assert status == 1
    # the launch ended normally: the next call runs to the end and is exact again
    h_ref, i_ref, h_p, i_p, status = _both(s, shape, wrs, bs, Ws, pws, h0)
    assert status == 0
    np.testing.assert_array_equal(i_p, i_ref)
    np.testing.assert_array_equal(h_p, h_ref)
    del keep, Ws, wrs, bs
    torch.cuda.empty_cache()
