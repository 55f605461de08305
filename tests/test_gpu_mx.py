"""GPU parity of the MX prefill path (MOE_F_MX_GEMM): MXFP4 weights on the fp8 x fp4 scaled matrix
cores, activations quantised to MXFP8 (OCP Microscaling Formats v1.0) before each contraction.

- moe_mxfp8_quantize against the oracle's quantiser, bit for bit: every E4M3 value and every tie
  at many block scales, fp32 subnormals, zero blocks, saturation, NaN / infinity blocks, bf16 rows.
- The two contractions separately, each from exact inputs.  Gate/up: the quantised SwiGLU output
  codes against the oracle's, which quantise the oracle's fp64 activations rounded to fp32.  The
  GPU's activations come from the scaled fp8 x fp4 MFMA, which does not sum its products at full
  fp32 precision: measured on gfx950, products far below the largest of their group are dropped
  (448 + 63 * 2^-9 returns 448.109 instead of 448.123; 1 + 63 * 2^-9 is exact).  We bound that
  sum's error by 2^-7 * sum |products| (at most 7 dropped terms per group of 8, each under 2^-10
  of the group's largest), carried through silu.  Where an activation lies that close to an E4M3
  rounding midpoint, or a block maximum that close to a power of two, both codes are correct and
  the GPU may differ, by at most that error plus one grid step; everywhere else the codes must be
  equal, and at most 2% of them may differ at all.  Down projection: fed the oracle's own codes,
  against the oracle's down projection of them, to the layer tolerance.
- The whole layer and the grouped FFN: routing bit for bit, the rms error against the quantising
  oracle below 1% and a tenth of the MX layer's own error against the exact layer (reported).
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


def _gpu_quantize(v: np.ndarray, dtype=torch.float32):
    x = torch.from_numpy(np.ascontiguousarray(v)).to("cuda")
    if dtype == torch.bfloat16:
        x = x.view(torch.bfloat16) if v.dtype == np.int16 else x.to(torch.bfloat16)
    rows, K = x.shape
    codes = torch.empty((rows, K), dtype=torch.uint8, device="cuda")
    scales = torch.empty((rows, K // 32), dtype=torch.uint8, device="cuda")
    moe.mxfp8_quantize(x, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def _e4m3_values() -> np.ndarray:
    b = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    return b.astype(np.float64)  # 0 .. 448


def test_mxfp8_quantize_bit_exact_fp32():
    rng = np.random.default_rng(11)
    pos = _e4m3_values()
    mids = (pos[:-1] + pos[1:]) / 2
    base = np.concatenate([pos, mids, -pos, -mids])
    blocks = []
    # every E4M3 value and tie under 2^e for e in a wide range: the block maximum 256 * 2^e fixes
    # the scale, so each element is a plain rounding (or its tie) at that scale
    for e in (-135, -120, -60, -9, -1, 0, 1, 7, 60, 110):
        vals = (base * 2.0 ** e).astype(np.float32)
        n = (len(vals) + 30) // 31
        blk = np.zeros((n, 32), np.float32)
        blk[:, 0] = np.float32(256.0 * 2.0 ** e)
        flat = blk[:, 1:].reshape(-1)
        flat[: len(vals)] = vals
        blk[:, 1:] = flat.reshape(n, 31)
        blocks.append(blk)
    # random magnitudes and signs, including values that saturate (block max just under 2^k)
    g = rng.standard_normal((512, 32)) * 2.0 ** rng.integers(-40, 40, (512, 1))
    blocks.append(g.astype(np.float32))
    sat = np.full((4, 32), 500.0, np.float32) * np.array([[1.0], [-1.0], [1e-20], [3e20]], np.float32)
    blocks.append(sat)
    blocks.append(np.zeros((2, 32), np.float32))
    sub = (rng.standard_normal((4, 32)) * 1e-40).astype(np.float32)  # fp32 subnormals
    blocks.append(sub)
    bad = rng.standard_normal((3, 32)).astype(np.float32)
    bad[0, 3], bad[1, 31], bad[2, 0] = np.nan, np.inf, -np.inf
    blocks.append(bad)
    v = np.ascontiguousarray(np.concatenate(blocks))
    c_ref, s_ref = oracle.mxfp8_quantize(v)
    c, s = _gpu_quantize(v)
    np.testing.assert_array_equal(s, s_ref)
    zero = (v == 0)  # +0 and -0 quantise to the same value; the sign of a zero code is free
    np.testing.assert_array_equal(c[~zero], c_ref[~zero])
    assert np.all((c[zero] & 0x7F) == 0)


def test_mxfp8_quantize_bit_exact_bf16_rows():
    x = mi.host_x(mi.spec("c3", T=64))  # bf16 bit patterns [64, 4096]
    c_ref, s_ref = oracle.mxfp8_quantize(np.ascontiguousarray((x.astype(np.uint32) << 16).view(np.float32)))
    c, s = _gpu_quantize(x.view(np.int16), torch.bfloat16)
    np.testing.assert_array_equal(s, s_ref)
    np.testing.assert_array_equal(c, c_ref)


SMALL = [
    mi.LayerSpec("mx_ragged", 257, 256, 128, 12, 2, 0, 0, "bf16", "mxfp4", 1.0, 0.0, 0.05, seed=23),
    mi.LayerSpec("mx_shared", 64, 256, 128, 8, 8, 1, 128, "bf16", "mxfp4", 1.0, 0.0, 0.05, seed=24),
    mi.LayerSpec("mx_shared_wide", 300, 384, 256, 16, 4, 1, 384, "bf16", "mxfp4", 1.0, 0.0, 0.05, seed=25),
    # K multiples of 512: the kernels fetch each row's scales 16 bytes at a time
    mi.LayerSpec("mx_k512", 160, 512, 512, 8, 2, 1, 1024, "bf16", "mxfp4", 1.0, 0.0, 0.05, seed=26),
]


def _deq(codes, sc):
    return oracle.mxfp4_dequant(codes.reshape(-1, codes.shape[-1]), sc.reshape(-1, sc.shape[-1])).astype(
        np.float64).reshape(*codes.shape[:-1], -1)


def _mx_values(codes, scales):
    v = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()
    return v * np.repeat(2.0 ** (scales.astype(np.float64) - 127), 32, axis=-1)


def _undecided(a_f64, xq_rows, w13, f):
    """Elements of the fp64 activation rows [R, f] whose MXFP8 code an fp32 evaluation may
    legitimately flip: within the bound of the fp32 sums of a rounding midpoint (or, for a whole
    block, of a power-of-two maximum).  xq_rows [R, d] are the quantised inputs, w13 [R, 2f, d] (or
    [2f, d]) the gate/up weights of each row."""
    gam = 2.0 ** -7 + (xq_rows.shape[1] + 2) * 2.0 ** -24
    if w13.ndim == 2:
        w13 = np.broadcast_to(w13, (xq_rows.shape[0],) + w13.shape)
    h = np.einsum("rnd,rd->rn", w13, xq_rows)
    habs = np.einsum("rnd,rd->rn", np.abs(w13), np.abs(xq_rows))
    g, u = h[:, :f], h[:, f:]
    sg = 1.0 / (1.0 + np.exp(-g))
    dsilu = sg * (1.0 + g * (1.0 - sg))
    da = np.abs(dsilu * u) * gam * habs[:, :f] + np.abs(g * sg) * gam * habs[:, f:] + 8 * 2.0 ** -24 * np.abs(a_f64)
    a = a_f64.astype(np.float32).astype(np.float64)
    R = a.shape[0]
    blk = np.abs(a).reshape(R, f // 32, 32)
    dab = da.reshape(R, f // 32, 32)
    amax = blk.max(axis=2, keepdims=True)
    lg = np.floor(np.log2(np.where(amax > 0, amax, 1.0)))
    X = 2.0 ** np.clip(lg - 8, -127, 127)
    q = blk / X
    lq = np.floor(np.log2(np.where(q > 0, q, 1.0)))
    step = np.where(q >= 2.0 ** -6, 2.0 ** (lq - 3), 2.0 ** -9)
    frac = q / step - np.floor(q / step)
    near = np.abs(frac - 0.5) * step * X <= dab
    damax = np.take_along_axis(dab, np.argmax(blk, axis=2)[..., None], axis=2)
    p2 = 2.0 ** lg
    bnear = (np.abs(amax - p2) <= damax) | (np.abs(2 * p2 - amax) <= damax)
    return (near.reshape(R, f), np.broadcast_to(bnear, blk.shape).reshape(R, f), bnear[..., 0],
            (step * X).reshape(R, f), da)


def _dev_weights(w, sh):
    return {k: dev(v) for k, v in w.items()}, ({k: dev(v) for k, v in sh.items()} if sh is not None else None)


def _rel_rms(a, b):
    return float(np.sqrt(np.mean((a - b) ** 2) / np.mean(b ** 2)))


def _routing(s, x, wr, b):
    l32, _ = oracle.router_logits(s, x, wr, b)
    idx, g = oracle.topk(s, l32)
    c, o, p, iv = oracle.permute(s, idx)
    return idx, g, o, p, iv


@pytest.mark.parametrize("s", SMALL, ids=lambda s: s.name)
def test_mx_gate_up_codes_match_oracle(s):
    x, wr, b, _ = margin_x(s)
    w = mi.host_experts(s)
    sh = mi.host_experts(s, shared=True) if s.n_shared else None
    wd, shd = _dev_weights(w, sh)
    idx, g, o, p, iv = _routing(s, x, wr, b)
    a, ash = oracle.swiglu_act(s, x, p, o, w, sh, flags=oracle.MX_GEMM)
    rows_a = [a] + ([ash] if sh is not None else [])
    P, fs = s.T * s.k, s.f_shared if s.n_shared else 0
    n_codes = P * s.f + s.T * fs
    codes = torch.empty(n_codes, dtype=torch.uint8, device="cuda")
    scales = torch.empty(n_codes // 32, dtype=torch.uint8, device="cuda")
    moe.mx_gate_up(moe.make_shape(s), dev(x), dev(p), dev(o), moe.make_weights(wd, shd), codes, scales)
    torch.cuda.synchronize()
    codes, scales = codes.cpu().numpy(), scales.cpu().numpy()
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    xc, xs = oracle.mxfp8_quantize(xf)
    xq = _mx_values(xc, xs)
    W13 = _deq(w["w13"], w["w13_scale"])
    slot_e = np.searchsorted(o, np.arange(P), side="right") - 1
    parts = [(a, s.f, codes[:P * s.f].reshape(P, s.f), scales[:P * s.f // 32].reshape(P, s.f // 32),
              xq[p // s.k], W13[slot_e])]
    if sh is not None:
        parts.append((ash, fs, codes[P * s.f:].reshape(s.T, fs), scales[P * s.f // 32:].reshape(s.T, fs // 32), xq,
                      _deq(sh["w13"], sh["w13_scale"])[0]))
    total_diff = 0
    for act, f, gc, gs, xr, w13 in parts:
        rc, rs = oracle.mxfp8_quantize(act.astype(np.float32))
        near, bnear_el, bnear, step, da = _undecided(act, xr, w13, f)
        # scales: equal except where the block maximum is undecided
        assert np.all((gs == rs) | bnear), f"{int(((gs != rs) & ~bnear).sum())} decided block scales differ"
        same_scale = np.repeat(gs == rs, 32, axis=1)
        gv, rv = _mx_values(gc, gs), _mx_values(rc, rs)
        diff = gv != rv  # by value: a -0 code equals a +0 code
        # codes under an equal scale: equal except undecided elements, and then one grid step apart
        bad = diff & same_scale & ~near & ~bnear_el
        assert not bad.any(), f"{int(bad.sum())} decided codes differ (of {int(diff.sum())} differing)"
        moved = np.abs(gv - rv)
        far = diff & same_scale & (moved > 1.0001 * (step + da))
        if far.any():
            r, c = np.argwhere(far)[0]
            raise AssertionError(f"{int(far.sum())} undecided codes moved by more than one grid step, e.g. row {r} "
                                 f"col {c}: a {act[r, c]:.9g}, gpu {gv[r, c]:.9g}, oracle {rv[r, c]:.9g}, "
                                 f"step {step[r, c]:.6g}, block scale byte {int(gs[r, c // 32])}")
        total_diff += int(diff.sum())
    print(f"{s.name}: {total_diff} of {n_codes} activation codes differ, all at undecided roundings")
    assert total_diff <= max(8, n_codes // 50)


@pytest.mark.parametrize("s", SMALL, ids=lambda s: s.name)
def test_mx_down_on_oracle_codes(s):
    x, wr, b, _ = margin_x(s)
    w = mi.host_experts(s)
    sh = mi.host_experts(s, shared=True) if s.n_shared else None
    wd, shd = _dev_weights(w, sh)
    idx, g, o, p, iv = _routing(s, x, wr, b)
    a, ash = oracle.swiglu_act(s, x, p, o, w, sh, flags=oracle.MX_GEMM)
    ys_ref, ysh_ref = oracle.grouped_ffn(s, x, p, o, w, sh, flags=oracle.MX_GEMM)
    rc, rs = oracle.mxfp8_quantize(a.astype(np.float32))
    codes, scales = [rc.reshape(-1)], [rs.reshape(-1)]
    if sh is not None:
        shc, shs = oracle.mxfp8_quantize(ash.astype(np.float32))
        codes.append(shc.reshape(-1))
        scales.append(shs.reshape(-1))
    P = s.T * s.k
    ys = torch.empty((P, s.d), dtype=torch.bfloat16, device="cuda")
    ysh = torch.empty((s.T, s.d), dtype=torch.bfloat16, device="cuda") if sh is not None else None
    moe.mx_down(moe.make_shape(s), dev(np.concatenate(codes)), dev(np.concatenate(scales)), dev(o),
                moe.make_weights(wd, shd), ys, ysh)
    torch.cuda.synchronize()
    assert_close(host(ys), ys_ref, what=f"{s.name} MX down (routed)")
    if sh is not None:
        assert_close(host(ysh), ysh_ref, what=f"{s.name} MX down (shared)")


@pytest.mark.parametrize("s", SMALL, ids=lambda s: s.name)
def test_mx_layer_small_against_quantising_oracle(s):
    x, wr, b, _ = margin_x(s)
    w = mi.host_experts(s)
    sh = mi.host_experts(s, shared=True) if s.n_shared else None
    wd, shd = _dev_weights(w, sh)
    ref = oracle.layer_forward(s, x, wr, b, w, sh, flags=oracle.MX_GEMM)
    exact = oracle.layer_forward(s, x, wr, b, w, sh)
    res = moe.layer_forward(s, dev(x), dev(wr), dev(b), wd, shd, flags=moe.F_MX_GEMM)  # T > 32: MFMA path
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(res["topk_idx"]), ref["topk_idx"])
    got = host(res["out"])
    err_q, err_x = _rel_rms(got, ref["out"]), _rel_rms(got, exact["out"])
    print(f"{s.name}: rms error vs quantising oracle {err_q:.2e}, vs exact layer {err_x:.2e}")
    assert err_q < 1e-2 and err_q < 0.1 * err_x


def test_mx_grouped_ffn_and_forced_gemm_at_small_T():
    s = SMALL[1].with_T(20)  # T <= 32: the flag takes effect with MOE_F_FORCE_GEMM
    x, wr, b, _ = margin_x(s)
    w, sh = mi.host_experts(s), mi.host_experts(s, shared=True)
    wd, shd = _dev_weights(w, sh)
    l32, _ = oracle.router_logits(s, x, wr, b)
    idx, g = oracle.topk(s, l32)
    c, o, p, iv = oracle.permute(s, idx)
    ys_ref, ysh_ref = oracle.grouped_ffn(s, x, p, o, w, sh, flags=oracle.MX_GEMM)
    shape = moe.make_shape(s, flags=moe.F_MX_GEMM | moe.F_FORCE_GEMM)
    ys = torch.empty((s.T * s.k, s.d), dtype=torch.bfloat16, device="cuda")
    ysh = torch.empty((s.T, s.d), dtype=torch.bfloat16, device="cuda")
    moe.grouped_ffn(shape, dev(x), dev(p), dev(o), moe.make_weights(wd, shd), ys, ysh)
    torch.cuda.synchronize()
    assert _rel_rms(host(ys), ys_ref) < 1e-2 and _rel_rms(host(ysh), ysh_ref) < 1e-2
    # the decode kernels ignore the flag: T <= 32 without FORCE_GEMM is the exact layer
    ref = oracle.layer_forward(s, x, wr, b, w, sh)
    res = moe.layer_forward(s, dev(x), dev(wr), dev(b), wd, shd, flags=moe.F_MX_GEMM)
    torch.cuda.synchronize()
    assert_close(host(res["out"]), ref["out"], what="flag ignored by decode")


def test_mx_partial_layers_merge():
    """The expert-mask partial layer (f1) on the MX path: complementary halves add up to the full
    MX layer (both through the GPU), and each half matches the oracle's masked MX layer."""
    s = SMALL[2]
    x, wr, b, _ = margin_x(s)
    w, sh = mi.host_experts(s), mi.host_experts(s, shared=True)
    wd, shd = _dev_weights(w, sh)
    W = moe.make_weights(wd, shd)
    mask_a = (np.random.default_rng(3).random(s.E + 1) < 0.5).astype(np.uint8)
    mask_b = (1 - mask_a).astype(np.uint8)
    ref_a = oracle.layer_forward(s, x, wr, b, w, sh, flags=oracle.MX_GEMM, expert_mask=mask_a)["out"]
    out_bf = torch.empty((s.T, s.d), dtype=torch.bfloat16, device="cuda")
    moe.layer_forward_masked_raw(moe.make_shape(s, flags=moe.F_MX_GEMM), dev(x), dev(wr), dev(b), W, dev(mask_a),
                                 out_bf)
    torch.cuda.synchronize()
    assert _rel_rms(host(out_bf), ref_a) < 1e-2
    moe.layer_forward_masked_raw(moe.make_shape(s, flags=moe.F_MX_GEMM | moe.F_ACCUMULATE), dev(x), dev(wr), dev(b),
                                 W, dev(mask_b), out_bf)
    torch.cuda.synchronize()
    full = oracle.layer_forward(s, x, wr, b, w, sh, flags=oracle.MX_GEMM)["out"]
    assert _rel_rms(host(out_bf), full) < 1e-2


def test_mx_prefill_c3_full_size():
    """E = 256, k = 6, d = 4096, f = 2048 at T = 8192 in the bench's launch configuration: routing
    on every token bit for bit, the layer on sampled tokens against the quantising oracle."""
    s = mi.spec("c3", T=8192)
    x, wr, b, _ = margin_x(s)
    wd = mi.device_experts(s)
    res = moe.layer_forward(s, dev(x), dev(wr), dev(b), wd, None, flags=moe.F_MX_GEMM)
    torch.cuda.synchronize()
    l32, _ = oracle.router_logits(s, x, wr, b)
    ref_idx, _ = oracle.topk(s, l32)
    np.testing.assert_array_equal(host(res["topk_idx"]), ref_idx)
    sample = np.sort(np.random.default_rng(4).choice(s.T, size=24, replace=False))
    sample[0], sample[-1] = 0, s.T - 1
    xs = np.ascontiguousarray(x[sample])
    l32s, _ = oracle.router_logits(s, xs, wr, b)
    idx_s, g_s = oracle.topk(s, l32s)
    need = sorted(set(idx_s.reshape(-1).tolist()))
    w = mi.host_experts(s, experts=need)
    remap = np.full(s.E, -1, np.int64)
    remap[need] = np.arange(len(need))
    idx_c = remap[idx_s].astype(np.int32)
    sc = mi.LayerSpec(s.name, len(sample), s.d, s.f, len(need), s.k, 0, 0, s.act, s.wt, s.sigma_x, s.sigma_w,
                      s.sigma_r)
    c, o, p, iv = oracle.permute(sc, idx_c)
    ys, _ = oracle.grouped_ffn(sc, xs, p, o, w, None, flags=oracle.MX_GEMM)
    ref = oracle.combine(sc, ys, iv, idx_c, g_s, None)
    ys_x, _ = oracle.grouped_ffn(sc, xs, p, o, w, None)
    exact = oracle.combine(sc, ys_x, iv, idx_c, g_s, None)
    got = host(res["out"])[sample]
    err_q, err_x = _rel_rms(got, ref), _rel_rms(got, exact)
    assert err_q < 1e-2 and err_q < 0.1 * err_x
    print(f"c3 MX prefill: rms error vs quantising oracle {_rel_rms(got, ref):.2e}, "
          f"vs exact layer {_rel_rms(got, exact):.2e}")
