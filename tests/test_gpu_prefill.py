"""GPU parity of the prefill path (grouped MFMA GEMM, MFMA router logits) against the oracle.

Small shapes are compared element by element over every output (ragged last tiles, several
m-tiles per expert, experts with no tokens).  The full-size prefill workloads (bf16 128-expert
top-8 + shared at T=4096, uniform and Zipf-skewed; MXFP4 256-expert top-6 at T=8192) run in the
same launch configuration as the bench: routing is checked bit for bit on every token, and the
layer output on a sample of tokens that the oracle evaluates one by one (tokens are independent
rows of the layer, so layer(x)[sample] = layer(x[sample])).
"""
from __future__ import annotations

import numpy as np
import pytest

import moe_inputs as mi
import oracle
from _gpu import dev, host, margin_x
from _helpers import assert_close

torch = pytest.importorskip("torch")
moe = pytest.importorskip("sparse_mixture_experts_16_amd")

pytestmark = pytest.mark.gpu

SMALL = [
    mi.LayerSpec("g_bf16", 333, 256, 128, 16, 4, 1, 192, "bf16", "bf16", 1.0, 0.05, 0.05, seed=21),
    mi.LayerSpec("g_bf16_noshared", 200, 512, 192, 24, 3, 0, 0, "bf16", "bf16", 1.0, 0.05, 0.05, seed=22),
    mi.LayerSpec("g_mxfp4", 257, 256, 128, 12, 2, 0, 0, "bf16", "mxfp4", 1.0, 0.0, 0.05, seed=23),
    mi.LayerSpec("g_mxfp4_shared", 64, 256, 128, 8, 8, 1, 128, "bf16", "mxfp4", 1.0, 0.0, 0.05, seed=24),
]


def _dev_weights(w, sh):
    return {k: dev(v) for k, v in w.items()}, ({k: dev(v) for k, v in sh.items()} if sh is not None else None)


@pytest.mark.parametrize("s", SMALL, ids=lambda s: s.name)
def test_layer_forward_gemm_small(s):
    x, wr, b, _ = margin_x(s)
    w = mi.host_experts(s)
    sh = mi.host_experts(s, shared=True) if s.n_shared else None
    wd, shd = _dev_weights(w, sh)
    ref = oracle.layer_forward(s, x, wr, b, w, sh)
    res = moe.layer_forward(s, dev(x), dev(wr), dev(b), wd, shd)  # T > 32: MFMA path
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(res["topk_idx"]), ref["topk_idx"])
    assert_close(host(res["out"]), ref["out"], what=s.name)


@pytest.mark.parametrize("s", SMALL[:3], ids=lambda s: s.name)
def test_grouped_ffn_gemm_small(s):
    x, wr, b, _ = margin_x(s)
    w = mi.host_experts(s)
    sh = mi.host_experts(s, shared=True) if s.n_shared else None
    wd, shd = _dev_weights(w, sh)
    l32, _ = oracle.router_logits(s, x, wr, b)
    idx, g = oracle.topk(s, l32)
    c, o, p, iv = oracle.permute(s, idx)
    ys_ref, ysh_ref = oracle.grouped_ffn(s, x, p, o, w, sh)
    shape = moe.make_shape(s)
    ys = torch.empty((s.T * s.k, s.d), dtype=torch.bfloat16, device="cuda")
    ysh = torch.empty((s.T, s.d), dtype=torch.bfloat16, device="cuda") if s.n_shared else None
    moe.grouped_ffn(shape, dev(x), dev(p), dev(o), moe.make_weights(wd, shd), ys, ysh)
    torch.cuda.synchronize()
    assert_close(host(ys), ys_ref, what="y_sorted (gemm)")
    if sh is not None:
        assert_close(host(ysh), ysh_ref, what="y_shared (gemm)")


@pytest.mark.parametrize("name,T", [("c1", 16), ("c3", 8), ("c3", 32)])
def test_forced_gemm_and_gemv_agree_with_oracle(name, T):
    s = mi.spec(name, T=T)
    x, wr, b, _ = margin_x(s)
    w = mi.host_experts(s)
    sh = mi.host_experts(s, shared=True) if s.n_shared else None
    wd, shd = _dev_weights(w, sh)
    ref = oracle.layer_forward(s, x, wr, b, w, sh)
    for flag in (moe.F_FORCE_GEMM, moe.F_FORCE_GEMV):
        res = moe.layer_forward(s, dev(x), dev(wr), dev(b), wd, shd, flags=flag)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(res["topk_idx"]), ref["topk_idx"])
        assert_close(host(res["out"]), ref["out"], what=f"{name} T={T} flag={flag}")


def _full_size_case(name, T, n_sample=48, seed=0):
    s = mi.spec(name, T=T)
    x, wr, b, _ = margin_x(s)
    # GPU: weights generated in device memory; oracle: the same bytes generated on the host.
    wd = mi.device_experts(s)
    shd = mi.device_experts(s, shared=True) if s.n_shared else None
    res = moe.layer_forward(s, dev(x), dev(wr), dev(b), wd, shd)
    torch.cuda.synchronize()
    l32, _ = oracle.router_logits(s, x, wr, b)
    ref_idx, _ = oracle.topk(s, l32)
    np.testing.assert_array_equal(host(res["topk_idx"]), ref_idx)
    counts = np.bincount(ref_idx.reshape(-1), minlength=s.E)
    rng = np.random.default_rng(seed)
    sample = np.sort(rng.choice(s.T, size=n_sample, replace=False))
    sample[0], sample[-1] = 0, s.T - 1  # first and last token (last m-tile tails)
    xs = np.ascontiguousarray(x[sample])
    need = sorted(set(ref_idx[sample].reshape(-1).tolist()))
    w = mi.host_experts(s, experts=need)
    remap = np.full(s.E, -1, np.int64)
    remap[need] = np.arange(len(need))
    # Oracle on the sampled tokens with the needed experts only: route with all E experts,
    # then evaluate the selected experts from the compacted weight set.
    sh = mi.host_experts(s, shared=True) if s.n_shared else None
    l32s, _ = oracle.router_logits(s, xs, wr, b)
    idx_s, g_s = oracle.topk(s, l32s)
    idx_c = remap[idx_s].astype(np.int32)
    sc = mi.LayerSpec(s.name, len(sample), s.d, s.f, len(need), s.k, s.n_shared, s.f_shared, s.act, s.wt,
                      s.sigma_x, s.sigma_w, s.sigma_r)
    c, o, p, iv = oracle.permute(sc, idx_c)
    ys, ysh = oracle.grouped_ffn(sc, xs, p, o, w, sh)
    ref = oracle.combine(sc, ys, iv, idx_c, g_s, ysh)
    got = host(res["out"])[sample]
    assert_close(got, ref, what=f"{name} sampled out")
    return counts


def test_prefill_c2_full_size():
    counts = _full_size_case("c2", 4096)
    assert counts.sum() == 4096 * 8 and (counts > 0).all()


def test_prefill_c2_skew_full_size():
    counts = _full_size_case("c2_skew", 4096)
    assert counts.sum() == 4096 * 8
    assert counts.max() > 4 * counts.mean()  # the Zipf prior concentrates the load


def test_prefill_c3_full_size():
    counts = _full_size_case("c3", 8192, n_sample=32)
    assert counts.sum() == 8192 * 6
