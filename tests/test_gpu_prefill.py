"""GPU parity of the prefill path (grouped MFMA GEMM, MFMA router logits) against the oracle.

Small shapes are compared element by element over every output (ragged last tiles, several
m-tiles per expert, experts with no tokens, 128- and 256-column down tiles, 128 x 256 and
128 x 512 gate/up tiles with and without a shared group).  The full-size prefill workloads run in
the same launch configuration as the bench, routing checked bit for bit on every token: the bf16
128-expert top-8 + shared layer at T=4096 (uniform and Zipf-skewed) on every output, the MXFP4
256-expert top-6 layer at T=8192 on every token that sits at the first or last row of an m-tile
of some expert (tokens are independent rows of the layer, so layer(x)[sample] = layer(x[sample])
and the oracle evaluates the sample with only the experts it selects).
"""
from __future__ import annotations

import numpy as np
import pytest

import moe_inputs as mi
import oracle
from _gpu import dev, host, margin_x, oracle_on_tokens, tile_boundary_tokens
from _helpers import assert_close, assert_literal

torch = pytest.importorskip("torch")
moe = pytest.importorskip("sparse_mixture_experts_16_amd")

pytestmark = pytest.mark.gpu

SMALL = [
    mi.LayerSpec("g_bf16", 333, 256, 128, 16, 4, 1, 192, "bf16", "bf16", 1.0, 0.05, 0.05, seed=21),
    mi.LayerSpec("g_bf16_noshared", 200, 512, 192, 24, 3, 0, 0, "bf16", "bf16", 1.0, 0.05, 0.05, seed=22),
    mi.LayerSpec("g_mxfp4", 257, 256, 128, 12, 2, 0, 0, "bf16", "mxfp4", 1.0, 0.0, 0.05, seed=23),
    mi.LayerSpec("g_mxfp4_shared", 64, 256, 128, 8, 8, 1, 128, "bf16", "mxfp4", 1.0, 0.0, 0.05, seed=24),
    # d_model not a multiple of 256: the down projection's 128-column tiles
    mi.LayerSpec("g_bf16_d192", 140, 192, 128, 8, 2, 1, 64, "bf16", "bf16", 1.0, 0.05, 0.05, seed=27),
    mi.LayerSpec("g_bf16_d320", 97, 320, 192, 12, 3, 1, 128, "bf16", "bf16", 1.0, 0.05, 0.05, seed=28),
    # MXFP4 with d_ff and shared d_ff multiples of 256: the 128 x 512 gate/up tiles, shared group
    # included; with d_model a multiple of 256 too, the down projection's MXFP8 correction plane
    mi.LayerSpec("g_mxfp4_f256_shared256", 150, 256, 256, 8, 2, 1, 256, "bf16", "mxfp4", 1.0, 0.0, 0.05, seed=29),
    mi.LayerSpec("g_mxfp4_f256_shared512", 70, 384, 256, 10, 3, 1, 512, "bf16", "mxfp4", 1.0, 0.0, 0.05, seed=30),
    # gate/up stage lengths: d_model not a multiple of 64 keeps bf16 weights on the 128-row tiles
    # with 32-element stages; MXFP4 with d_ff a multiple of 256 but d_model not of 128 keeps the
    # 128 x 512 tiles on 32-element stages (the others above take the long stages)
    mi.LayerSpec("g_bf16_d224", 120, 224, 128, 8, 2, 1, 128, "bf16", "bf16", 1.0, 0.05, 0.05, seed=31),
    mi.LayerSpec("g_mxfp4_f256_d160", 90, 160, 256, 8, 2, 0, 0, "bf16", "mxfp4", 1.0, 0.0, 0.05, seed=32),
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


# the step call with bf16 y_sorted: bf16 weights, MXFP4 with a bf16 correction plane (d_ff 128), and
# MXFP4 with the MXFP8 correction plane (d_model, d_ff and shared d_ff multiples of 256)
@pytest.mark.parametrize("s", SMALL[:3] + SMALL[6:7], ids=lambda s: s.name)
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


def _full_size_case(name, T, all_tokens):
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
    tokens = np.arange(T) if all_tokens else tile_boundary_tokens(ref_idx, s.E, T, s.n_shared)
    print(f"{name}: comparing {len(tokens)} of {T} tokens element by element", flush=True)
    ref = oracle_on_tokens(s, x, wr, b, tokens)
    got, want = host(res["out"])[tokens], ref["out"]
    rms = float(np.sqrt(np.mean(want * want)))
    ratio = np.abs(got - want) / (1e-2 * rms + 2e-2 * np.abs(want))
    print(f"{name}: largest error / bound {ratio.max():.3f}; {int((ratio > 0.5).sum())} elements above half the bound",
          flush=True)
    assert_close(got, want, what=f"{name} out")
    if name.startswith("c2"):
        assert_literal(got, want, what=f"{name} out")
    return counts


def test_prefill_c2_full_size():
    """Every one of the 4096 tokens."""
    counts = _full_size_case("c2", 4096, all_tokens=True)
    assert counts.sum() == 4096 * 8 and (counts > 0).all()


def test_prefill_c2_skew_full_size():
    """Every one of the 4096 tokens."""
    counts = _full_size_case("c2_skew", 4096, all_tokens=True)
    assert counts.sum() == 4096 * 8
    assert counts.max() > 4 * counts.mean()  # the Zipf prior concentrates the load


def test_prefill_c3_full_size():
    """The tokens at the first and last row of every m-tile of every expert."""
    counts = _full_size_case("c3", 8192, all_tokens=False)
    assert counts.sum() == 8192 * 6


# An E8M0 scale byte of 0xFF makes its whole 32-element block NaN (OCP MX rule).  Planted in one
# gate/up block of expert 0 and one down block of expert 1, the NaN must reach exactly the outputs
# the oracle's does: every column of the tokens routed to expert 0, column 5 of those routed to
# expert 1.  (The GEMM's expansion relies on the scaled convert returning NaN under the infinite
# scale that byte decodes to.)
@pytest.mark.parametrize("s", [SMALL[2], SMALL[6]], ids=lambda s: s.name)
def test_gemm_mxfp4_nan_scale_block(s):
    x, wr, b, _ = margin_x(s)
    w = mi.host_experts(s)
    sh = mi.host_experts(s, shared=True) if s.n_shared else None
    w["w13_scale"] = w["w13_scale"].copy()
    w["w2_scale"] = w["w2_scale"].copy()
    w["w13_scale"][0, 3, 1] = 0xFF
    w["w2_scale"][1, 5, 0] = 0xFF
    wd, shd = _dev_weights(w, sh)
    ref = oracle.layer_forward(s, x, wr, b, w, sh)
    res = moe.layer_forward(s, dev(x), dev(wr), dev(b), wd, shd)
    torch.cuda.synchronize()
    out = host(res["out"])
    np.testing.assert_array_equal(host(res["topk_idx"]), ref["topk_idx"])
    assert np.isnan(ref["out"]).any() and not np.isnan(ref["out"]).all()
    assert_close(out, ref["out"], what=s.name + " with NaN scale blocks")
