"""The seeded input generator: host C implementation against a pure-Python transcription of
its published definition (SplitMix64), distribution checks, and (GPU) device == host bytes."""
from __future__ import annotations

import numpy as np
import pytest

import moe_inputs as mi

M64 = (1 << 64) - 1


def _mix(z):
    z ^= z >> 30
    z = (z * 0xBF58476D1CE4E5B9) & M64
    z ^= z >> 27
    z = (z * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def _word(key, i):
    return _mix((key + (i + 1) * 0x9E3779B97F4A7C15) & M64)


def test_splitmix64_reference_sequence():
    # SplitMix64 seeded with 0: the first output is mix(0x9E3779B97F4A7C15) = 0xE220A8397B1DCDAF,
    # the widely published first value of Vigna's splitmix64.c with state 0.
    assert _word(0, 0) == 0xE220A8397B1DCDAF
    for key in (0, 1, 1234567, 0xDEADBEEFCAFEBABE):
        for i in (0, 1, 2, 1000, 2 ** 40):
            assert mi.word(key, i) == _word(key, i)
    assert mi.derive(5, 9) == _mix(5 ^ _mix((9 + 0x9E3779B97F4A7C15) & M64))


def test_normal_values_are_exact_irwin_hall():
    key = 42
    c = mi.normal_scale(0.02)
    got = mi.host_normal(100, key, 0.02, "f32")
    for i in range(100):
        r = _word(key, i)
        s = sum((r >> (16 * q)) & 0xFFFF for q in range(4)) - 131070
        assert got[i] == np.float32(np.float32(s) * np.float32(c))


def test_normal_distribution_moments():
    v = mi.host_normal(400_000, 7, 1.0, "f32").astype(np.float64)
    assert abs(v.mean()) < 0.01
    assert abs(v.std() - 1.0) < 0.01
    assert np.abs(v).max() <= 2 * np.sqrt(3.0) + 1e-6


def test_bf16_is_round_to_nearest_even_of_f32():
    f = mi.host_normal(10_000, 9, 1.0, "f32")
    b = mi.host_normal(10_000, 9, 1.0, "bf16")
    u = f.view(np.uint32).astype(np.uint64)
    rne = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    np.testing.assert_array_equal(b, rne)
    # and the bf16 value is the nearest to the f32 value
    up = (b.astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.abs(up.astype(np.float64) - f) <= np.abs(f) * 2.0 ** -8 + 1e-30)


def test_scale_bytes_in_range_and_uniform():
    a = np.empty(90_000, np.uint8)
    mi._load_host().mg_fill_scale_bytes(a.ctypes.data, a.size, 3, 119, 127, 0)
    assert a.min() == 119 and a.max() == 127
    h = np.bincount(a - 119, minlength=9)
    assert np.all(np.abs(h / a.size - 1 / 9) < 0.01)


def test_expert_substreams_regenerate_alone():
    s = mi.LayerSpec("t", 4, 64, 32, 6, 2, 0, 0, "bf16", "mxfp4", 1.0, 0.0, 0.02)
    all_w = mi.host_experts(s)
    some = mi.host_experts(s, experts=[4, 1])
    for k in all_w:
        np.testing.assert_array_equal(some[k][0], all_w[k][4])
        np.testing.assert_array_equal(some[k][1], all_w[k][1])


def test_x_rows_resample_independently():
    s = mi.spec("c1", T=4)
    x0 = mi.host_x(s)
    att = np.array([0, 1, 0, 0])
    x1 = mi.host_x(s, attempts=att)
    np.testing.assert_array_equal(x0[[0, 2, 3]], x1[[0, 2, 3]])
    assert not np.array_equal(x0[1], x1[1])


def test_zipf_bias_is_log_rank_permutation():
    s = mi.spec("c2_skew")
    b = mi.router_bias(s)
    r = np.exp(-b.astype(np.float64) / 1.1)
    np.testing.assert_allclose(np.sort(r), np.arange(1, s.E + 1), rtol=1e-5)


@pytest.mark.gpu
def test_device_generator_matches_host():
    import torch
    for name in ("c0", "c3"):
        s = mi.spec(name)
        dev = mi.device_experts(s)
        host = mi.host_experts(s, experts=[0, s.E - 1])
        torch.cuda.synchronize()
        for k, v in dev.items():
            d = v.cpu()
            if d.dtype == torch.bfloat16:
                d = d.view(torch.int16)
            d = d.numpy()
            np.testing.assert_array_equal(d[0].view(host[k].dtype), host[k][0])
            np.testing.assert_array_equal(d[-1].view(host[k].dtype), host[k][1])
    s = mi.spec("c1")
    dev = mi.device_experts(s, shared=True)
    host = mi.host_experts(s, shared=True)
    torch.cuda.synchronize()
    for k, v in dev.items():
        np.testing.assert_array_equal(v.cpu().view(torch.int16).numpy().view(np.uint16), host[k])
