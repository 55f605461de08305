"""Pins of the CPU oracle against what the mathematics and public definitions fix.

Every test here checks the oracle against something other than itself: the OCP MX
specification's E2M1 table, an independent bit-field decoding, brute-force sorting,
numpy/scipy library routines (float64 matmul, stable argsort, softmax), closed forms
and invariants of the layer (sparse == dense with zeroed gates, k = E with identical
experts == one dense FFN, sum of counts == T*k, exact merge of partial sums).
CPU only.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

import moe_inputs as mi
import oracle
from _helpers import assert_close, bf16_to_f64, ref_select, to_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------------------------
# MXFP4 dequantisation (test iv of the layer's acceptance list)
# ---------------------------------------------------------------------------------------------
def _golden_e2m1():
    vals = {}
    with open(os.path.join(GOLDEN, "e2m1_ocp_mx_v1.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            vals[int(c)] = float(v)
    assert len(vals) == 16
    return vals


def _pack(codes):
    """Pack a row of 4-bit codes (even element -> low nibble)."""
    codes = np.asarray(codes, np.uint8)
    return (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)


def test_e2m1_matches_ocp_table_at_unit_scale():
    gold = _golden_e2m1()
    codes = np.array([c for c in range(16)] * 2, np.uint8)  # 32 elements = one scale block
    out = oracle.mxfp4_dequant(_pack(codes)[None, :], np.array([[127]], np.uint8))[0]
    for j, c in enumerate(codes):
        assert out[j] == gold[int(c)], (c, out[j], gold[int(c)])
        assert math.copysign(1.0, out[j]) == math.copysign(1.0, gold[int(c)]), ("sign of zero", c)


def _independent_e2m1(code: int, scale: int) -> np.float32:
    """Decode from the bit fields (sign, 2-bit exponent with bias 1, 1-bit mantissa) with exact
    rationals, then scale by 2^(scale-127) and round once to fp32 (overflow -> inf)."""
    if scale == 255:
        return np.float32(np.nan)
    sign = -1 if code & 8 else 1
    e = (code >> 1) & 3
    m = code & 1
    mag = Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
    v = mag * Fraction(2) ** (scale - 127)
    with np.errstate(over="ignore"):
        f = np.float32(float(v)) if v < Fraction(2) ** 1000 else np.float32(np.inf)
    if f == 0:
        return np.float32(-0.0) if sign < 0 else np.float32(0.0)
    return np.float32(sign * f)


def test_mxfp4_dequant_exhaustive_codes_by_scales():
    """All 16 codes x 256 scale bytes, bit for bit (NaN for scale 0xFF, -0.0 for code 8)."""
    codes = np.array(list(range(16)) * 2, np.uint8)  # 32 elements per row: one scale block
    packed = np.tile(_pack(codes), (256, 1))
    scales = np.arange(256, dtype=np.uint8)[:, None]
    out = oracle.mxfp4_dequant(packed, scales)
    for s in range(256):
        for j in range(32):
            want = _independent_e2m1(int(codes[j]), s)
            got = out[s, j]
            if np.isnan(want):
                assert np.isnan(got), (s, j)
            else:
                assert got.view(np.uint32) == want.view(np.uint32), (s, int(codes[j]), got, want)


def test_mxfp4_nibble_order_and_scale_blocks():
    # Byte 0x21: element 0 = code 1 (0.5), element 1 = code 2 (1.0).
    row = np.zeros(32, np.uint8)
    row[0] = 0x21
    out = oracle.mxfp4_dequant(row[None, :], np.array([[127, 127]], np.uint8))[0]
    assert out[0] == 0.5 and out[1] == 1.0 and np.all(out[2:] == 0)
    # Scales apply per 32 consecutive elements of a row.
    codes = np.full(64, 2, np.uint8)  # all 1.0
    out = oracle.mxfp4_dequant(_pack(codes)[None, :], np.array([[126, 129]], np.uint8))[0]
    assert np.all(out[:32] == 0.5) and np.all(out[32:] == 4.0)
    # Rows use their own scale rows.
    out = oracle.mxfp4_dequant(np.tile(_pack(codes), (2, 1)), np.array([[127, 127], [128, 128]], np.uint8))
    assert np.all(out[0] == 1.0) and np.all(out[1] == 2.0)


# ---------------------------------------------------------------------------------------------
# MXFP8 quantisation (OCP Microscaling Formats v1.0: E4M3 elements, one E8M0 scale per 32)
# ---------------------------------------------------------------------------------------------
def _torch_e4m3_round(v: np.ndarray) -> np.ndarray:
    """Independent element rounding: torch's cast to float8_e4m3fn (round to nearest even;
    it has no saturation, so callers keep |v| <= 448)."""
    torch = pytest.importorskip("torch")
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_mxfp8_element_rounding_matches_torch_float8_cast():
    """Blocks whose largest magnitude is 256 have shared scale 2^0, so each code is the plain
    E4M3 rounding of the value: every E4M3 value, every midpoint between neighbours (ties go to
    the even code), subnormal midpoints and random values, with both signs."""
    pos = _torch_e4m3(np.arange(0, 127, dtype=np.uint8)).astype(np.float64)  # 0 .. 448, increasing
    mids = (pos[:-1] + pos[1:]) / 2
    rnd = np.random.default_rng(3).uniform(0, 448, 4000)
    vals = np.concatenate([pos, mids, rnd, (np.arange(0, 17) + 0.5) * 2.0 ** -9])
    vals = np.concatenate([vals, -vals]).astype(np.float32)
    vals = vals[np.abs(vals) <= 256]  # keep 256 the block maximum
    n = (len(vals) + 30) // 31
    blocks = np.zeros((n, 32), np.float32)
    blocks[:, 0] = 256.0
    flat = blocks[:, 1:].reshape(-1)
    flat[: len(vals)] = vals
    blocks[:, 1:] = flat.reshape(n, 31)
    codes, scales = oracle.mxfp8_quantize(blocks)
    assert np.all(scales == 127)
    want = _torch_e4m3_round(blocks)
    zero = blocks == 0  # -0 and +0 carry the same value
    assert np.array_equal(codes[~zero], want[~zero])
    assert np.all(codes[zero] & 0x7F == 0)


def test_mxfp8_shared_exponent_and_saturation_landmarks():
    """The shared scale is floor(log2 amax) - 8 (8 = E4M3's largest exponent), clamped to the
    E8M0 range; magnitudes above 448 after scaling clamp to 448 (0x7E / 0xFE)."""
    cases = [  # (amax, scale byte)
        (1.0, 119), (1.999, 119), (2.0, 120), (448.0, 127), (511.9, 127), (512.0, 128),
        (2.0 ** -126, 0), (2.0 ** -130, 0), (3.0e38, 127 + 127 - 8), (0.75, 118),
    ]
    for amax, want in cases:
        blk = np.zeros((1, 32), np.float32)
        blk[0, 5] = np.float32(amax)
        c, sc = oracle.mxfp8_quantize(blk)
        assert int(sc[0, 0]) == want, (amax, int(sc[0, 0]), want)
    blk = np.zeros((1, 32), np.float32)
    c, sc = oracle.mxfp8_quantize(blk)
    assert sc[0, 0] == 0 and np.all(c == 0)
    # saturation: amax in [448, 512) keeps scale 2^0, so 460 and 500 exceed the largest normal
    blk = np.array([[460.0, -500.0, 448.0, 447.0] + [0.0] * 28], np.float32)
    c, sc = oracle.mxfp8_quantize(blk)
    assert sc[0, 0] == 127 and list(c[0, :4]) == [0x7E, 0xFE, 0x7E, 0x7E]
    # a value just under a power of two still takes the lower exponent
    blk = np.array([[np.nextafter(np.float32(4.0), np.float32(0.0))] + [0.0] * 31], np.float32)
    _, sc = oracle.mxfp8_quantize(blk)
    assert sc[0, 0] == 127 + 1 - 8


def test_mxfp8_blocks_and_rows_are_independent():
    rng = np.random.default_rng(5)
    v = rng.standard_normal((3, 96)).astype(np.float32)
    c0, s0 = oracle.mxfp8_quantize(v)
    assert c0.shape == (3, 96) and s0.shape == (3, 3)
    v2 = v.copy()
    v2[1, 32:64] *= 1000.0
    c1, s1 = oracle.mxfp8_quantize(v2)
    keep = np.ones((3, 96), bool)
    keep[1, 32:64] = False
    assert np.array_equal(c0[keep], c1[keep])
    assert s1[1, 1] == s0[1, 1] + 9 or s1[1, 1] == s0[1, 1] + 10
    assert np.array_equal(np.delete(s0.reshape(-1), 4), np.delete(s1.reshape(-1), 4))


def _np_mx(v: np.ndarray) -> np.ndarray:
    """MXFP8 quantise-dequantise of fp32 rows, written from the specification in numpy with
    torch's float8 cast for the element rounding."""
    v = np.ascontiguousarray(v, np.float32)
    blk = v.reshape(v.shape[0], -1, 32).astype(np.float64)
    amax = np.abs(blk).max(axis=2, keepdims=True)
    e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8, -127)
    e = np.clip(e, -127, 127)
    q = np.clip(blk / 2.0 ** e, -448.0, 448.0).astype(np.float32)
    deq = _torch_e4m3(_torch_e4m3_round(q)).astype(np.float64) * 2.0 ** e
    return deq.reshape(v.shape)


# ---------------------------------------------------------------------------------------------
# The MX path's contractions: the fp8 x fp4 matrix core's grouped, truncated sum
# ---------------------------------------------------------------------------------------------
_E2M1 = {0.0: 0, 0.5: 1, 1.0: 2, 1.5: 3, 2.0: 4, 3.0: 5, 4.0: 6, 6.0: 7}


def _e4m3_code(v: float) -> int:
    """E4M3 code of an exactly representable value (torch's float8 cast, checked exact)."""
    torch = pytest.importorskip("torch")
    c = int(torch.tensor([v], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)[0])
    assert float(_torch_e4m3(np.array([c], np.uint8))[0]) == v, v
    return c


def _row(xv, wv, K=64, xs=127, ws=127):
    """MXFP8 / MXFP4 operands from element values (zeros elsewhere) and per-block scale bytes."""
    xc = np.zeros(K, np.uint8)
    wn = np.full(K, _E2M1[1.0], np.uint8)
    for i, v in xv.items():
        xc[i] = _e4m3_code(v)
    for i, v in wv.items():
        wn[i] = _E2M1[abs(v)] | (8 if v < 0 else 0)
    wc = (wn[0::2] | (wn[1::2] << 4)).astype(np.uint8)
    xsb = np.full(K // 32, xs, np.uint8) if np.isscalar(xs) else np.asarray(xs, np.uint8)
    wsb = np.full(K // 32, ws, np.uint8) if np.isscalar(ws) else np.asarray(ws, np.uint8)
    return xc, xsb, wc, wsb


def test_mx_dot_without_truncation_is_the_plain_dot():
    """Products that all share the exponent sum 0 and have at most 4 fractional bits lose nothing
    to the 13-bit window, and their sums are exact in fp32: the result is numpy's dot."""
    rng = np.random.default_rng(81)
    for K in (32, 64, 256):
        xv = rng.integers(8, 16, K) / 8.0 * rng.choice([-1.0, 1.0], K)   # E4M3 values in [1, 2)
        wv = rng.choice([1.0, 1.5], K) * rng.choice([-1.0, 1.0], K)       # E2M1 values of exponent 0
        args = _row(dict(enumerate(xv)), dict(enumerate(wv)), K)
        assert oracle.mx_dot(*args) == float(np.dot(xv, wv))


def test_mx_dot_block_scales_and_nibble_order():
    """Each 32-element block's product is multiplied by 2^(sx - 127) * 2^(sw - 127); element 2i of
    the weight row is the low nibble of byte i."""
    xv = {0: 1.5, 33: 1.25, 70: -1.0}
    wv = {0: 3.0, 33: 1.5, 70: 4.0}
    got = oracle.mx_dot(*_row(xv, wv, K=96, xs=[127, 129, 125], ws=[128, 126, 127]))
    want = 1.5 * 3.0 * 2.0 ** 1 + 1.25 * 1.5 * 2.0 ** (2 - 1) + (-1.0) * 4.0 * 2.0 ** -2
    assert got == want
    xc, xs, wc, ws = _row({1: 1.0}, {1: 6.0, 0: 0.5})  # the odd element sits in the high nibble
    assert wc[0] == (_E2M1[0.5] | (_E2M1[6.0] << 4)) and oracle.mx_dot(xc, xs, wc, ws) == 6.0


def test_mx_dot_alignment_window_closed_forms():
    """A product bit below 2^(E - 13) is dropped, E = the group's largest e(x) + e(w)."""
    t = 2.0 ** -9  # the smallest E4M3 subnormal (exponent -6, mantissa 1/8)
    for p in range(9):
        got = oracle.mx_dot(*_row({0: 2.0 ** p, **{i: t for i in range(1, 8)}}, {}))
        assert got == (2.0 ** p + 7 * t if p <= 4 else 2.0 ** p), p  # 2^-9 >= 2^(p - 13) iff p <= 4
    # one small term with bits at 2^-6 and 2^-9: the 2^-9 bit goes first, then the whole term
    for p in range(9):
        v = 1.125 * 2.0 ** -6
        got = oracle.mx_dot(*_row({0: 2.0 ** p, 1: v}, {}))
        want = 2.0 ** p + (v if p <= 4 else (2.0 ** -6 if p <= 7 else 0.0))
        assert got == want, p
    # the anchor is the exponent sum, not the product's own magnitude: 3.5 * 6 = 21 has
    # e = 1 + 2 = 3 (keeps 2^-10), 4 * 4 = 16 has e = 4 (drops it)
    for xb, wb, kept in ((3.5, 6.0, True), (7.0, 3.0, True), (14.0, 1.5, True), (4.0, 4.0, False),
                         (7.0, 4.0, False), (16.0, 0.5, False), (8.0, 1.5, True)):
        small = {i: t for i in range(1, 8)}
        got = oracle.mx_dot(*_row({0: xb, **small}, {0: wb, **{i: 0.5 for i in range(1, 8)}}))
        assert got == xb * wb + (7 * t * 0.5 if kept else 0.0), (xb, wb)


def test_mx_dot_truncates_toward_zero_per_group():
    t = 2.0 ** -9
    assert oracle.mx_dot(*_row({0: 32.0, 1: -t}, {})) == 32.0
    assert oracle.mx_dot(*_row({0: 32.0, 1: -3 * t}, {})) == 32.0 - 2.0 ** -8
    assert oracle.mx_dot(*_row({0: 32.0, 1: 3 * t}, {})) == 32.0 + 2.0 ** -8
    assert oracle.mx_dot(*_row({0: -32.0, 1: t}, {})) == -32.0
    assert oracle.mx_dot(*_row({0: -32.0, 1: -3 * t}, {})) == -32.0 - 2.0 ** -8
    assert oracle.mx_dot(*_row({0: 32.0, 1: -1.125 * 2.0 ** -6}, {})) == 32.0 - 2.0 ** -6
    # a cancelling pair still sets the window: the small terms beside it are dropped
    assert oracle.mx_dot(*_row({0: 256.0, 1: -256.0, **{i: t for i in range(2, 8)}}, {})) == 0.0
    # groups are 8 consecutive elements: the small terms of the next group keep their bits
    for g0 in (8, 16, 32, 56):
        got = oracle.mx_dot(*_row({0: 256.0, **{i: t for i in range(g0, g0 + 8)}}, {}))
        assert got == 256.0 + 8 * t, g0
    assert oracle.mx_dot(*_row({4: 256.0, **{i: t for i in range(8) if i != 4}}, {})) == 256.0


def test_mx_dot_zero_products_do_not_set_the_window():
    """A zero weight beside a large activation leaves the group's other products alone, while a
    0.5 weight (the E2M1 subnormal) counts with exponent 0: 32 * 0.5 sets E = 5."""
    t = 2.0 ** -9
    small = {i: t for i in range(2, 8)}
    assert oracle.mx_dot(*_row({0: 448.0, 1: 1.0, **small}, {0: 0.0})) == 1.0 + 6 * t
    assert oracle.mx_dot(*_row({0: 448.0, 1: 1.0, **small}, {0: -0.0})) == 1.0 + 6 * t
    assert oracle.mx_dot(*_row({0: 32.0, 1: 1.0, **small}, {0: 0.5})) == 16.0 + 1.0
    assert oracle.mx_dot(*_row({0: 16.0, 1: 1.0, **small}, {0: 0.5})) == 8.0 + 1.0 + 6 * t
    assert oracle.mx_dot(*_row({}, {})) == 0.0


def test_mx_dot_rounds_the_accumulator_once_per_64_elements():
    """Within one 64-element step the group sums and the accumulator are added exactly and
    rounded to fp32 once: 2^18 + two groups of 2^-6 gives 2^18 + 2^-5 (each 2^-6 alone would be
    a tie, rounded to even); across steps the accumulator is rounded each time."""
    t = 2.0 ** -9
    xc, xs, wc, ws = _row({0: 256.0, **{i: t for i in range(32, 48)}}, {0: 4.0}, K=64, xs=[135, 127])
    assert oracle.mx_dot(xc, xs, wc, ws) == 2.0 ** 18 + 2.0 ** -5
    xc, xs, wc, ws = _row({0: 256.0, **{i: t for i in range(64, 72)}, **{i: t for i in range(128, 136)}}, {0: 4.0},
                          K=192, xs=[135, 127, 127, 127, 127, 127])
    assert oracle.mx_dot(xc, xs, wc, ws) == 2.0 ** 18


def test_mx_dot_error_bound_on_random_rows():
    """Against the exact dot: per group at most 7 truncations, each under 2^(E - 13) of the
    block scales, plus the fp32 accumulator's rounding once per step."""
    rng = np.random.default_rng(82)
    e4m3 = np.array([_torch_e4m3(np.array([c], np.uint8))[0] for c in range(0x7F)], np.float64)
    for _ in range(40):
        K = 256
        xc = rng.integers(0, 0x7F, K).astype(np.uint8) | (rng.integers(0, 2, K) << 7).astype(np.uint8)
        wn = rng.integers(0, 16, K).astype(np.uint8)
        xs = rng.integers(119, 128, K // 32).astype(np.uint8)
        ws = rng.integers(119, 128, K // 32).astype(np.uint8)
        wc = (wn[0::2] | (wn[1::2] << 4)).astype(np.uint8)
        xv = np.where(xc & 0x80, -1.0, 1.0) * e4m3[xc & 0x7F]
        wv = np.where(wn & 8, -1.0, 1.0) * np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])[wn & 7]
        sc = np.repeat(2.0 ** (xs.astype(np.float64) - 127 + ws.astype(np.float64) - 127), 32)
        prods = xv * wv * sc
        exact = float(prods.sum())
        ex = np.where((xc & 0x78) > 0, ((xc >> 3) & 15).astype(np.int64) - 7, -6)
        ew = np.where((wn & 6) > 0, ((wn >> 1) & 3).astype(np.int64) - 1, 0)
        E = (ex + ew).reshape(-1, 8).max(axis=1)
        trunc_bound = float((7 * 2.0 ** (E - 13) * sc[::8]).sum())
        acc_bound = (K // 64) * 2.0 ** -24 * float(np.abs(prods).sum())
        assert abs(oracle.mx_dot(xc, xs, wc, ws) - exact) <= trunc_bound + acc_bound


def test_mx_gemm_layer_is_the_composition_of_its_steps():
    """MOE_REF_MX_GEMM layer: routing unchanged; x quantised to MXFP8 (the quantiser pinned above),
    gate/up rows as mx_dot, SwiGLU, the fp32-rounded activation quantised to MXFP8, down rows as
    mx_dot, the gate-weighted combine; composed here in numpy from those pinned steps."""
    s = mi.LayerSpec("mx_small", 4, 64, 64, 4, 2, 1, 32, "bf16", "mxfp4", 1.0, 0.0, 0.05, seed=72)
    x = mi.host_x(s)
    wr, b = mi.host_router(s)
    w, sh = mi.host_experts(s), mi.host_experts(s, shared=True)
    ref = oracle.layer_forward(s, x, wr, b, w, sh, flags=oracle.MX_GEMM)
    plain = oracle.layer_forward(s, x, wr, b, w, sh)
    np.testing.assert_array_equal(ref["topk_idx"], plain["topk_idx"])
    xc, xs = oracle.mxfp8_quantize(bf16_to_f64(x).astype(np.float32))

    def ffn(w13, w13s, w2, w2s, t, f):
        h = np.array([oracle.mx_dot(xc[t], xs[t], w13[j], w13s[j]) for j in range(2 * f)])
        a = (h[:f] / (1.0 + np.exp(-h[:f])) * h[f:]).astype(np.float32)
        ac, asc = oracle.mxfp8_quantize(a[None, :])
        return np.array([oracle.mx_dot(ac[0], asc[0], w2[i], w2s[i]) for i in range(s.d)])

    want = np.zeros((s.T, s.d))
    for t in range(s.T):
        for j in range(s.k):
            e = int(ref["topk_idx"][t, j])
            want[t] += ref["topk_w"][t, j] * ffn(w["w13"][e], w["w13_scale"][e], w["w2"][e], w["w2_scale"][e], t, s.f)
        want[t] += ffn(sh["w13"][0], sh["w13_scale"][0], sh["w2"][0], sh["w2_scale"][0], t, s.f_shared)
    np.testing.assert_allclose(ref["out"], want, rtol=1e-12, atol=1e-12 * np.abs(want).max())
    # the quantisation is visible: the MX layer differs from the exact one by a few percent
    err = np.sqrt(np.mean((ref["out"] - plain["out"]) ** 2) / np.mean(plain["out"] ** 2))
    assert 1e-3 < err < 0.2, err


def test_swiglu_act_is_the_grouped_ffn_intermediate():
    """moe_ref_swiglu_act: numpy silu(Wg x) * (Wu x) per sorted slot (plain), and under the MX
    flag the down projection of its MXFP8-rounded rows gives the grouped FFN's output."""
    s = mi.LayerSpec("act_small", 5, 64, 64, 4, 2, 1, 32, "bf16", "mxfp4", 1.0, 0.0, 0.05, seed=73)
    x = mi.host_x(s)
    wr, b = mi.host_router(s)
    w, sh = mi.host_experts(s), mi.host_experts(s, shared=True)
    l32, _ = oracle.router_logits(s, x, wr, b)
    idx, _ = oracle.topk(s, l32)
    _, off, perm, _ = oracle.permute(s, idx)

    def deq(codes, sc):
        return oracle.mxfp4_dequant(codes.reshape(-1, codes.shape[-1]), sc.reshape(-1, sc.shape[-1])).astype(
            np.float64).reshape(*codes.shape[:-1], -1)

    W13, W2 = deq(w["w13"], w["w13_scale"]), deq(w["w2"], w["w2_scale"])
    S13 = deq(sh["w13"], sh["w13_scale"])[0]
    xf = bf16_to_f64(x)
    a, ash = oracle.swiglu_act(s, x, perm, off, w, sh)
    for i in range(s.T * s.k):
        e = int(np.searchsorted(off, i, side="right") - 1)
        h = W13[e] @ xf[perm[i] // s.k]
        np.testing.assert_allclose(a[i], h[:s.f] / (1.0 + np.exp(-h[:s.f])) * h[s.f:], rtol=1e-12, atol=1e-15)
    for t in range(s.T):
        h = S13 @ xf[t]
        fs = s.f_shared
        np.testing.assert_allclose(ash[t], h[:fs] / (1.0 + np.exp(-h[:fs])) * h[fs:], rtol=1e-12, atol=1e-15)
    am, _ = oracle.swiglu_act(s, x, perm, off, w, sh, flags=oracle.MX_GEMM)
    ys, _ = oracle.grouped_ffn(s, x, perm, off, w, sh, flags=oracle.MX_GEMM)
    for i in range(s.T * s.k):
        e = int(np.searchsorted(off, i, side="right") - 1)
        ac, asc = oracle.mxfp8_quantize(am[i].astype(np.float32)[None, :])
        want = [oracle.mx_dot(ac[0], asc[0], w["w2"][e][r], w["w2_scale"][e][r]) for r in range(s.d)]
        np.testing.assert_array_equal(ys[i], want)


def test_mx_gemm_flag_needs_mxfp4_weights():
    s = mi.spec("c0")
    x = mi.host_x(s)
    wr, b = mi.host_router(s)
    with pytest.raises(ValueError):
        oracle.layer_forward(s, x, wr, b, mi.host_experts(s), flags=oracle.MX_GEMM)


# ---------------------------------------------------------------------------------------------
# NVFP4 dequantisation: E2M1 x FP8 E4M3 block scale (16 elements) x fp32 tensor scale
# ---------------------------------------------------------------------------------------------
def _torch_e4m3(b: np.ndarray) -> np.ndarray:
    """Independent decode of E4M3 bytes: torch's float8_e4m3fn dtype."""
    torch = pytest.importorskip("torch")
    t = torch.from_numpy(np.ascontiguousarray(b, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy()


def test_e4m3_landmarks_of_the_ocp_fp8_spec():
    with open(os.path.join(GOLDEN, "e4m3_ocp_fp8_v1.txt")) as fh:
        rows = [l.split() for l in fh if l.strip() and not l.startswith("#")]
    b = np.array([int(r[0], 16) for r in rows], np.uint8)
    got = oracle.e4m3_to_f32(b)
    for (hx, v), g in zip(rows, got):
        want = float(v)
        if math.isnan(want):
            assert math.isnan(g), hx
        else:
            assert g == want and math.copysign(1.0, g) == math.copysign(1.0, want), (hx, g, want)


def test_e4m3_all_bytes_against_torch_float8():
    b = np.arange(256, dtype=np.uint8)
    got, want = oracle.e4m3_to_f32(b), _torch_e4m3(b)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok].view(np.uint32), want[ok].view(np.uint32))


def test_nvfp4_dequant_exhaustive_codes_by_scales():
    """All 16 codes x 256 scale bytes x a non-power-of-two tensor scale, bit for bit: the exact
    product E2M1 * E4M3 * g rounded once to fp32 (NaN for the E4M3 NaN bytes)."""
    gold = _golden_e2m1()
    g = 0.3
    codes = np.array(list(range(16)), np.uint8)             # 16 elements: one scale block
    packed = np.tile(_pack(codes), (256, 1))
    scales = np.arange(256, dtype=np.uint8)[:, None]
    out = oracle.nvfp4_dequant(packed, scales, g)
    sv = _torch_e4m3(np.arange(256, dtype=np.uint8)).astype(np.float64)
    g32 = float(np.float32(g))
    for s in range(256):
        for j in range(16):
            exact = Fraction(gold[j]) * Fraction(float(sv[s])) * Fraction(g32) if not np.isnan(sv[s]) else None
            if exact is None:
                assert np.isnan(out[s, j]), (s, j)
                continue
            want = np.float32(float(exact))  # exact rational -> nearest double -> fp32 (no double rounding: < 53 bits)
            assert out[s, j].view(np.uint32) == want.view(np.uint32) or (want == 0 and out[s, j] == 0), (s, j, out[s, j], want)


def test_nvfp4_scale_blocks_of_16_and_nibble_order():
    row = np.zeros(16, np.uint8)
    row[0] = 0x21  # element 0 = code 1 (0.5), element 1 = code 2 (1.0)
    out = oracle.nvfp4_dequant(row[None, :], np.array([[0x38, 0x38]], np.uint8), 1.0)[0]
    assert out[0] == 0.5 and out[1] == 1.0 and np.all(out[2:] == 0)
    codes = np.full(32, 2, np.uint8)  # all 1.0; scales 0.5 (0x30) then 2.0 (0x40)
    out = oracle.nvfp4_dequant(_pack(codes)[None, :], np.array([[0x30, 0x40]], np.uint8), 1.0)[0]
    assert np.all(out[:16] == 0.5) and np.all(out[16:] == 2.0)


def test_nvfp4_expert_ffn_matches_numpy_on_dequantised_weights():
    """The oracle's NVFP4 grouped FFN equals a float64 numpy SwiGLU over weights decoded
    independently (golden E2M1 table x torch's E4M3 x tensor scale)."""
    s = mi.LayerSpec("nv_small", 5, 64, 32, 4, 2, 1, 32, "bf16", "nvfp4", 1.0, 0.0, 0.05,
                     scale_lo=mi.NVFP4_SCALE_LO, scale_hi=mi.NVFP4_SCALE_HI, seed=71)
    x = mi.host_x(s)
    w = mi.host_experts(s)
    sh = mi.host_experts(s, shared=True)
    gold = _golden_e2m1()
    table = np.array([gold[c] for c in range(16)], np.float64)

    def deq(codes, sc, g):
        c = np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(*codes.shape[:-1], -1)
        sv = _torch_e4m3(sc).astype(np.float64)
        return table[c] * np.repeat(sv, 16, axis=-1) * float(np.float32(g))

    xf = bf16_to_f64(x)
    l32, _ = oracle.router_logits(s, x, *mi.host_router(s))
    idx, _ = oracle.topk(s, l32)
    _, off, perm, _ = oracle.permute(s, idx)
    ys, ysh = oracle.grouped_ffn(s, x, perm, off, w, sh)
    W13 = deq(w["w13"], w["w13_scale"], w["w13_gscale"])
    W2 = deq(w["w2"], w["w2_scale"], w["w2_gscale"])
    for i in range(s.T * s.k):
        e = int(np.searchsorted(off, i, side="right") - 1)
        want = _np_ffn(W13[e], W2[e], xf[perm[i] // s.k], s.f)
        np.testing.assert_allclose(ys[i], want, rtol=1e-12, atol=1e-14 * np.abs(want).max())
    S13 = deq(sh["w13"], sh["w13_scale"], sh["w13_gscale"])[0]
    S2 = deq(sh["w2"], sh["w2_scale"], sh["w2_gscale"])[0]
    for t in range(s.T):
        want = _np_ffn(S13, S2, xf[t], s.f_shared)
        np.testing.assert_allclose(ysh[t], want, rtol=1e-12, atol=1e-14 * np.abs(want).max())


# ---------------------------------------------------------------------------------------------
# Top-k selection and gates
# ---------------------------------------------------------------------------------------------
class _S:
    """Minimal shape object for direct oracle calls."""
    def __init__(self, **kw):
        self.T, self.d, self.f, self.E, self.k = 1, 8, 8, 8, 2
        self.n_shared, self.f_shared, self.act, self.wt = 0, 0, "f32", "f32"
        self.__dict__.update(kw)


def test_topk_exhaustive_ties_E8_k2():
    """Every logit pattern in {0,1,2}^8 (6561 rows) against a full stable sort by (-l, e)."""
    grid = np.array(np.meshgrid(*([np.arange(3)] * 8), indexing="ij")).reshape(8, -1).T.astype(np.float32)
    s = _S(E=8, k=2)
    idx, _ = oracle.topk(s, grid)
    for t in range(grid.shape[0]):
        assert list(idx[t]) == ref_select(grid[t], 2), (grid[t], idx[t])


@pytest.mark.parametrize("k", [1, 3, 8])
def test_topk_total_order_nan_and_signed_zero(k):
    rng = np.random.default_rng(7)
    specials = np.array([np.nan, 0.0, -0.0, np.inf, -np.inf, 1.0, -1.0], np.float32)
    rows = rng.choice(specials, size=(4000, 8)).astype(np.float32)
    s = _S(E=8, k=k)
    idx, _ = oracle.topk(s, rows)
    for t in range(rows.shape[0]):
        assert list(idx[t]) == ref_select(rows[t], k), (rows[t], idx[t])


def test_gates_sum_to_one_and_match_softmax_of_selected():
    rng = np.random.default_rng(1)
    l = rng.normal(size=(500, 128)).astype(np.float32)
    s = _S(E=128, k=8)
    idx, g = oracle.topk(s, l)
    np.testing.assert_allclose(g.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    sel = np.take_along_axis(l.astype(np.float64), idx.astype(np.int64), axis=1)
    np.testing.assert_allclose(g, scipy.special.softmax(sel, axis=1), rtol=1e-13, atol=0)
    assert np.all(np.diff(sel, axis=1) <= 0), "selection order must be descending logits"


def test_no_renorm_with_k_equal_E_is_full_softmax():
    rng = np.random.default_rng(2)
    l = rng.normal(size=(200, 16)).astype(np.float32)
    s = _S(E=16, k=16)
    idx, g = oracle.topk(s, l, flags=oracle.NO_RENORM)
    full = scipy.special.softmax(l.astype(np.float64), axis=1)
    np.testing.assert_allclose(g, np.take_along_axis(full, idx.astype(np.int64), axis=1), rtol=1e-13)
    # NO_RENORM with k < E: the selected entries of the full softmax (they no longer sum to 1).
    s2 = _S(E=16, k=4)
    idx2, g2 = oracle.topk(s2, l, flags=oracle.NO_RENORM)
    np.testing.assert_allclose(g2, np.take_along_axis(full, idx2.astype(np.int64), axis=1), rtol=1e-13)


# ---------------------------------------------------------------------------------------------
# Permute (test iii: counts sum to T*k)
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (16, 8, 2), (37, 128, 8), (300, 256, 6), (5, 4, 4)])
def test_permute_is_stable_counting_sort(T, E, k):
    rng = np.random.default_rng(T * 1000 + E)
    # Distinct experts per token, as top-k produces.
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    s = _S(E=E, k=k, T=T)
    counts, offsets, perm, inv = oracle.permute(s, idx)
    flat = idx.reshape(-1)
    assert counts.sum() == T * k
    np.testing.assert_array_equal(counts, np.bincount(flat, minlength=E))
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    np.testing.assert_array_equal(perm, np.argsort(flat, kind="stable"))
    np.testing.assert_array_equal(inv[perm], np.arange(T * k))
    assert sorted(perm.tolist()) == list(range(T * k))


def test_permute_skewed_all_tokens_one_expert():
    T, E, k = 50, 16, 1
    idx = np.full((T, k), 5, np.int32)
    counts, offsets, perm, inv = oracle.permute(_S(E=E, k=k, T=T), idx)
    assert counts[5] == T and counts.sum() == T
    np.testing.assert_array_equal(perm, np.arange(T))
    assert offsets[5] == 0 and offsets[6] == T and offsets[-1] == T


# ---------------------------------------------------------------------------------------------
# Router logits and expert FFN against numpy float64
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["c0", "c1"])
def test_router_logits_match_numpy_matmul(name):
    s = mi.spec(name, T=16)
    x = mi.host_x(s)
    wr, _ = mi.host_router(s)
    b = np.random.default_rng(0).normal(size=s.E).astype(np.float32)  # a nonzero bias must be added
    l32, l64 = oracle.router_logits(s, x, wr, b)
    want = to_f64(x) @ to_f64(wr).T + b.astype(np.float64)
    np.testing.assert_allclose(l64, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())
    # The fp32 logits are the fp64 value rounded once.
    np.testing.assert_array_equal(l32, l64.astype(np.float32))


def _np_ffn(w13, w2, xv, f):
    h = w13 @ xv
    g, u = h[:f], h[f:]
    return w2 @ (g / (1.0 + np.exp(-g)) * u)


@pytest.mark.parametrize("name", ["c0", "c1_small", "c3_small"])
def test_expert_ffn_matches_numpy(name):
    if name == "c0":
        s = mi.spec("c0")
    elif name == "c1_small":
        s = mi.LayerSpec("c1s", 6, 256, 96, 8, 3, 1, 64, "bf16", "bf16", 1.0, 0.02, 0.02)
    else:
        s = mi.LayerSpec("c3s", 5, 128, 64, 8, 2, 0, 0, "bf16", "mxfp4", 1.0, 0.0, 0.02)
    x = mi.host_x(s)
    wr, b = mi.host_router(s)
    w = mi.host_experts(s)
    sh = mi.host_experts(s, shared=True) if s.n_shared else None
    l32, _ = oracle.router_logits(s, x, wr, b)
    idx, _ = oracle.topk(s, l32)
    counts, offsets, perm, inv = oracle.permute(s, idx)
    ys, ysh = oracle.grouped_ffn(s, x, perm, offsets, w, sh)
    if s.wt == "mxfp4":
        E = s.E
        w13 = oracle.mxfp4_dequant(w["w13"].reshape(E * 2 * s.f, -1), w["w13_scale"].reshape(E * 2 * s.f, -1))
        w13 = w13.reshape(E, 2 * s.f, s.d).astype(np.float64)
        w2 = oracle.mxfp4_dequant(w["w2"].reshape(E * s.d, -1), w["w2_scale"].reshape(E * s.d, -1))
        w2 = w2.reshape(E, s.d, s.f).astype(np.float64)
    else:
        w13, w2 = to_f64(w["w13"]), to_f64(w["w2"])
    xf = to_f64(x)
    for i in range(s.T * s.k):
        p = perm[i]
        t, e = p // s.k, idx.reshape(-1)[p]
        assert offsets[e] <= i < offsets[e + 1]
        want = _np_ffn(w13[e], w2[e], xf[t], s.f)
        np.testing.assert_allclose(ys[i], want, rtol=1e-10, atol=1e-12 * max(np.abs(want).max(), 1e-300))
    if sh is not None:
        for t in range(s.T):
            want = _np_ffn(to_f64(sh["w13"][0]), to_f64(sh["w2"][0]), xf[t], s.f_shared)
            np.testing.assert_allclose(ysh[t], want, rtol=1e-10, atol=1e-12 * np.abs(want).max())


# ---------------------------------------------------------------------------------------------
# Layer invariants (tests i and ii of the acceptance list, and the exact partial-sum merge)
# ---------------------------------------------------------------------------------------------
def _small_layers():
    return [
        mi.spec("c0"),
        mi.LayerSpec("c1s", 9, 128, 64, 16, 4, 1, 48, "bf16", "bf16", 1.0, 0.02, 0.02, seed=77),
        mi.LayerSpec("c3s", 7, 128, 64, 12, 3, 0, 0, "bf16", "mxfp4", 1.0, 0.0, 0.02, seed=78),
    ]


@pytest.mark.parametrize("s", _small_layers(), ids=lambda s: s.name)
def test_sparse_equals_dense_with_zeroed_gates(s):
    """Test (i): the sparse layer equals evaluating all E experts densely with the gates of
    non-selected experts set to zero.  The dense side is numpy float64 written here
    (own selection by sorting, own softmax, own FFN), so only fp64 rounding differs."""
    x = mi.host_x(s)
    wr, b = mi.host_router(s)
    w = mi.host_experts(s)
    sh = mi.host_experts(s, shared=True) if s.n_shared else None
    ref = oracle.layer_forward(s, x, wr, b, w, sh)
    xf = to_f64(x)
    logits = (xf @ to_f64(wr).T + b.astype(np.float64)).astype(np.float32)
    if s.wt == "mxfp4":
        E = s.E
        w13 = oracle.mxfp4_dequant(w["w13"].reshape(E * 2 * s.f, -1), w["w13_scale"].reshape(E * 2 * s.f, -1)).reshape(E, 2 * s.f, s.d)
        w2 = oracle.mxfp4_dequant(w["w2"].reshape(E * s.d, -1), w["w2_scale"].reshape(E * s.d, -1)).reshape(E, s.d, s.f)
        w13, w2 = w13.astype(np.float64), w2.astype(np.float64)
    else:
        w13, w2 = to_f64(w["w13"]), to_f64(w["w2"])
    out = np.zeros((s.T, s.d))
    for t in range(s.T):
        sel = ref_select(logits[t], s.k)
        assert sel == list(ref["topk_idx"][t])
        gates = np.zeros(s.E)
        z = np.exp(logits[t][sel].astype(np.float64) - float(logits[t][sel[0]]))
        gates[sel] = z / z.sum()
        for e in range(s.E):  # dense over every expert, zero gates included
            out[t] += gates[e] * _np_ffn(w13[e], w2[e], xf[t], s.f)
        if sh is not None:
            out[t] += _np_ffn(to_f64(sh["w13"][0]), to_f64(sh["w2"][0]), xf[t], s.f_shared)
    assert_close(ref["out"], out, rel=1e-10, abs_of_rms=1e-12, what="sparse vs dense")


def test_k_equal_E_with_identical_experts_is_one_dense_ffn():
    """Test (ii): with k = E and all experts equal, gates sum to 1 and the layer is one FFN."""
    s = mi.LayerSpec("ident", 10, 64, 32, 8, 8, 0, 0, "f32", "f32", 0.5, 0.1, 0.1, seed=5)
    x = mi.host_x(s)
    wr, b = mi.host_router(s)
    w = mi.host_experts(s, experts=[0] * s.E)  # expert 0's weights, E times
    ref = oracle.layer_forward(s, x, wr, b, w)
    xf = to_f64(x)
    for t in range(s.T):
        want = _np_ffn(to_f64(w["w13"][0]), to_f64(w["w2"][0]), xf[t], s.f)
        np.testing.assert_allclose(ref["out"][t], want, rtol=1e-12, atol=1e-14 * np.abs(want).max())
    np.testing.assert_allclose(ref["topk_w"].sum(axis=1), 1.0, atol=1e-14)


@pytest.mark.parametrize("s", _small_layers(), ids=lambda s: s.name)
def test_split_sum_merges_exactly(s):
    """Partial sums over any split of the experts merge to the full layer (the exact merge of
    the q* policy's GPU and CPU partial results: dothoosh.com FreeToken article,
    "FreeToken architecture and the sparsity puzzle", mechanism 1)."""
    x = mi.host_x(s)
    wr, b = mi.host_router(s)
    w = mi.host_experts(s)
    sh = mi.host_experts(s, shared=True) if s.n_shared else None
    full = oracle.layer_forward(s, x, wr, b, w, sh)["out"]
    rng = np.random.default_rng(11)
    for _ in range(3):
        mask_a = (rng.random(s.E + 1) < 0.5).astype(np.uint8)
        mask_b = (1 - mask_a).astype(np.uint8)
        a = oracle.layer_forward(s, x, wr, b, w, sh, expert_mask=mask_a)["out"]
        # Accumulate the second part onto the first, as the merge does.
        ab = oracle.layer_forward(s, x, wr, b, w, sh, expert_mask=mask_b, flags=oracle.ACCUMULATE, out_init=a)["out"]
        assert_close(ab, full, rel=1e-12, abs_of_rms=1e-13, what="split-sum")


@pytest.mark.parametrize("T", [1, 4, 16])
def test_counts_sum_to_T_times_k_on_decode_config(T):
    s = mi.spec("c1", T=T)
    x = mi.host_x(s)
    wr, b = mi.host_router(s)
    l32, _ = oracle.router_logits(s, x, wr, b)
    idx, g = oracle.topk(s, l32)
    counts, offsets, perm, inv = oracle.permute(s, idx)
    assert counts.sum() == T * s.k
    assert all(len(set(r)) == s.k for r in idx.tolist())


# ---------------------------------------------------------------------------------------------
# Residual-stack glue
# ---------------------------------------------------------------------------------------------
def _all_bf16_finite():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = bf16_to_f64(bits)
    ok = np.isfinite(v)
    return np.sort(np.unique(v[ok]))


def _nearest_bf16_brute(v: float, table: np.ndarray) -> float:
    i = np.searchsorted(table, v)
    cands = [table[j] for j in (i - 1, i) if 0 <= j < len(table)]
    best = min(cands, key=lambda c: abs(c - v))
    ties = [c for c in cands if abs(c - v) == abs(best - v)]
    if len(ties) > 1:  # tie: the one with an even last mantissa bit
        ties = [c for c in ties if (np.float32(c).view(np.uint32) >> 16) & 1 == 0]
    return float(ties[0])


def test_rmsnorm_matches_closed_form_and_rounds_to_nearest_bf16():
    table = _all_bf16_finite()
    rng = np.random.default_rng(3)
    h = rng.normal(size=(4, 256)).astype(np.float32)
    x32 = oracle.rmsnorm(h, 1e-6, "f32")
    hf = h.astype(np.float64)
    want = hf / np.sqrt(np.mean(hf * hf, axis=1, keepdims=True) + 1e-6)
    np.testing.assert_array_equal(x32, want.astype(np.float32))
    xb = bf16_to_f64(oracle.rmsnorm(h, 1e-6, "bf16"))
    for t in range(4):
        for i in range(0, 256, 7):
            assert xb[t, i] == _nearest_bf16_brute(want[t, i], table), (t, i)


def test_stack_layer_is_residual_plus_layer_of_normed_input():
    s = mi.LayerSpec("stk", 3, 128, 64, 16, 3, 0, 0, "bf16", "mxfp4", 1.0, 0.0, 0.02, seed=91)
    rng = np.random.default_rng(4)
    h = rng.normal(size=(s.T, s.d)).astype(np.float32)
    wr, b = mi.host_router(s)
    w = mi.host_experts(s)
    x = oracle.rmsnorm(h, 1e-6, "bf16")
    lay = oracle.layer_forward(s, x, wr, b, w)
    h2 = h.copy()
    idx = oracle.stack_layer(s, h2, wr, b, w)
    np.testing.assert_array_equal(idx, lay["topk_idx"])
    np.testing.assert_array_equal(h2, (h.astype(np.float64) + lay["out"]).astype(np.float32))
    # Zero expert weights leave the residual stream unchanged.
    wz = {k: np.zeros_like(v) for k, v in w.items()}
    h3 = h.copy()
    oracle.stack_layer(s, h3, wr, b, wz)
    np.testing.assert_array_equal(h3, h)
