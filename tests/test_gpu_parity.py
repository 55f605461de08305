"""GPU parity: every C-ABI entry point against the CPU oracle on the same seeded inputs.

Integer outputs (top-k indices, counts, offsets, perm, inv_perm) must match bit for bit.
Floating outputs must satisfy, element by element,
    |gpu - oracle| <= 1e-2 * rms(oracle) + 2e-2 * |oracle|
(the layer's stated 1e-2 absolute / 2e-2 relative bounds, with the absolute part taken
relative to the output's rms because the configurations' outputs range from ~1e-5 to ~1e5).
Gates (softmax of fp32 logits) must agree to 1e-5 relative.
"""
from __future__ import annotations

import numpy as np
import pytest

import moe_inputs as mi
import oracle
from _gpu import dev, host, margin_x
from _helpers import assert_close, assert_literal, ref_select

torch = pytest.importorskip("torch")
moe = pytest.importorskip("sparse_mixture_experts_16_amd")

pytestmark = pytest.mark.gpu


def _weights(spec, layer=0):
    w = mi.host_experts(spec, layer)
    sh = mi.host_experts(spec, layer, shared=True) if spec.n_shared else None
    wd = {k: dev(v) for k, v in w.items()}
    shd = {k: dev(v) for k, v in sh.items()} if sh is not None else None
    return w, sh, wd, shd


DECODE_CASES = [("c0", 16), ("c1", 1), ("c1", 4), ("c1", 16), ("c3", 1), ("c3", 8), ("c3", 32)]


# ---------------------------------------------------------------------------------------------
# Router
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("E,k", [(8, 2), (128, 8), (256, 6), (64, 64), (1000, 3)])
def test_route_logits_in_exact_ties(E, k):
    """Integer-valued logits with many exact ties, NaN, +-0 and +-inf: the selection must follow
    the total order bit for bit."""
    rng = np.random.default_rng(E * 31 + k)
    T = 300
    vals = np.array([0.0, -0.0, 1.0, 2.0, -1.0, 3.0, np.nan, np.inf, -np.inf], np.float32)
    l = rng.integers(0, 4, size=(T, E)).astype(np.float32)
    l[T // 2:] = rng.choice(vals, size=(T - T // 2, E))
    s = mi.LayerSpec("r", T, 64, 64, E, k, 0, 0, "f32", "f32", 1, 1, 1)
    ref_idx, ref_w = oracle.topk(s, l)
    shape = moe.make_shape(s)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    lo = torch.empty((T, E), dtype=torch.float32, device="cuda")
    li = dev(l)
    moe.route(shape, None, None, None, idx, w, logits_in=li, logits_out=lo)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(idx), ref_idx)
    np.testing.assert_array_equal(host(lo).view(np.uint32), l.view(np.uint32))
    gw = host(w)
    fin = np.isfinite(ref_w)
    np.testing.assert_allclose(gw[fin], ref_w[fin], rtol=1e-5, atol=1e-7)
    assert np.array_equal(np.isnan(gw), np.isnan(ref_w))


@pytest.mark.parametrize("name,T", DECODE_CASES + [("c2", 4096), ("c3", 8192)])
def test_route_computed_logits(name, T):
    s = mi.spec(name, T=T)
    x, wr, b, _ = margin_x(s)
    l32, l64 = oracle.router_logits(s, x, wr, b)
    ref_idx, ref_w = oracle.topk(s, l32)
    shape = moe.make_shape(s)
    idx = torch.empty((T, s.k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, s.k), dtype=torch.float32, device="cuda")
    lo = torch.empty((T, s.E), dtype=torch.float32, device="cuda")
    moe.route(shape, dev(x), dev(wr), dev(b), idx, w, logits_out=lo)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(idx), ref_idx)
    assert_close(host(lo), l64, rel=1e-5, abs_of_rms=1e-5, what="logits")
    np.testing.assert_allclose(host(w), ref_w, rtol=2e-5, atol=1e-7)


# ---------------------------------------------------------------------------------------------
# Permute
# ---------------------------------------------------------------------------------------------
# (4099, 24, 1): just past the one-workgroup sort, a last chunk of 3 pairs (one wavefront's piece
# partly filled, the others empty); (4500, 7, 3): an odd expert count of many counts per thread
@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (16, 8, 2), (16, 128, 8), (32, 256, 6), (512, 128, 8),
                                   (4096, 128, 8), (8192, 256, 6), (3000, 1000, 7), (777, 16, 16),
                                   (4099, 24, 1), (4500, 7, 3)])
def test_permute_bit_exact(T, E, k):
    rng = np.random.default_rng(T + E + k)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    s = mi.LayerSpec("p", T, 64, 64, E, k, 0, 0, "bf16", "bf16", 1, 1, 1)
    c, o, p, iv = oracle.permute(s, idx)
    shape = moe.make_shape(s)
    out = [torch.full((n,), -7, dtype=torch.int32, device="cuda") for n in (E, E + 1, T * k, T * k)]
    moe.permute(shape, dev(idx), *out)
    torch.cuda.synchronize()
    for got, want in zip(out, (c, o, p, iv)):
        np.testing.assert_array_equal(host(got), want)


def test_permute_skewed_all_to_one_expert():
    T, E, k = 5000, 64, 1
    idx = np.full((T, k), 17, np.int32)
    s = mi.LayerSpec("p", T, 64, 64, E, k, 0, 0, "bf16", "bf16", 1, 1, 1)
    c, o, p, iv = oracle.permute(s, idx)
    out = [torch.empty((n,), dtype=torch.int32, device="cuda") for n in (E, E + 1, T * k, T * k)]
    moe.permute(moe.make_shape(s), dev(idx), *out)
    torch.cuda.synchronize()
    for got, want in zip(out, (c, o, p, iv)):
        np.testing.assert_array_equal(host(got), want)


# ---------------------------------------------------------------------------------------------
# MXFP4 dequantisation: all 16 codes x 256 scale bytes
# ---------------------------------------------------------------------------------------------
def test_mxfp4_dequant_table_bit_exact():
    codes = np.array(list(range(16)) * 2, np.uint8)
    packed = np.tile((codes[0::2] | (codes[1::2] << 4)).astype(np.uint8), (256, 1))
    scales = np.arange(256, dtype=np.uint8)[:, None].copy()
    ref = oracle.mxfp4_dequant(packed, scales)
    out = torch.empty((256, 32), dtype=torch.float32, device="cuda")
    moe.mxfp4_dequant(dev(packed), dev(scales), out)
    torch.cuda.synchronize()
    got = host(out)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    bad = np.nonzero((got.view(np.uint32) != ref.view(np.uint32)) & ~nan)
    assert bad[0].size == 0, f"mismatch at scale bytes {sorted(set(bad[0].tolist()))[:20]}"


# ---------------------------------------------------------------------------------------------
# Grouped FFN, combine, whole layer
# ---------------------------------------------------------------------------------------------
def _route_ref(s, x, wr, b):
    l32, _ = oracle.router_logits(s, x, wr, b)
    idx, g = oracle.topk(s, l32)
    c, o, p, iv = oracle.permute(s, idx)
    return idx, g, c, o, p, iv


@pytest.mark.parametrize("name,T", DECODE_CASES)
def test_grouped_ffn_and_combine(name, T):
    s = mi.spec(name, T=T)
    x, wr, b, _ = margin_x(s)
    w, sh, wd, shd = _weights(s)
    idx, g, c, o, p, iv = _route_ref(s, x, wr, b)
    ys_ref, ysh_ref = oracle.grouped_ffn(s, x, p, o, w, sh)
    shape = moe.make_shape(s)
    act = torch.float32 if s.act == "f32" else torch.bfloat16
    ys = torch.empty((T * s.k, s.d), dtype=act, device="cuda")
    ysh = torch.empty((T, s.d), dtype=act, device="cuda") if s.n_shared else None
    moe.grouped_ffn(shape, dev(x), dev(p), dev(o), moe.make_weights(wd, shd), ys, ysh)
    torch.cuda.synchronize()
    assert_close(host(ys), ys_ref, what="y_sorted")
    if s.n_shared:
        assert_close(host(ysh), ysh_ref, what="y_shared")
    # combine on the oracle's own expert outputs (rounded to the activation dtype)
    out = torch.empty((T, s.d), dtype=act, device="cuda")
    ys_in = torch.from_numpy(ys_ref).to(act).cuda()
    ysh_in = torch.from_numpy(ysh_ref).to(act).cuda() if s.n_shared else None
    moe.combine(shape, ys_in, dev(iv), dev(g.astype(np.float32)), ysh_in, out)
    torch.cuda.synchronize()
    ref = oracle.combine(s, ys_ref, iv, idx, g, ysh_ref)
    assert_close(host(out), ref, what="combine")


@pytest.mark.parametrize("name,T", DECODE_CASES)
def test_layer_forward_decode(name, T):
    s = mi.spec(name, T=T)
    x, wr, b, _ = margin_x(s)
    w, sh, wd, shd = _weights(s)
    ref = oracle.layer_forward(s, x, wr, b, w, sh)
    res = moe.layer_forward(s, dev(x), dev(wr), dev(b), wd, shd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(res["topk_idx"]), ref["topk_idx"])
    assert_close(host(res["out"]), ref["out"], what=f"{name} T={T} out")
    if name == "c1":
        assert_literal(host(res["out"]), ref["out"], what=f"{name} T={T} out")


@pytest.mark.parametrize("name,T", [("c0", 16), ("c1", 4), ("c3", 8)])
def test_layer_forward_accumulate_and_determinism(name, T):
    s = mi.spec(name, T=T)
    x, wr, b, _ = margin_x(s)
    w, sh, wd, shd = _weights(s)
    ref = oracle.layer_forward(s, x, wr, b, w, sh)
    r1 = moe.layer_forward(s, dev(x), dev(wr), dev(b), wd, shd)
    r2 = moe.layer_forward(s, dev(x), dev(wr), dev(b), wd, shd)
    torch.cuda.synchronize()
    assert torch.equal(r1["out"], r2["out"]), "two runs differ bitwise"
    resid = r1["out"].clone()
    r3 = moe.layer_forward(s, dev(x), dev(wr), dev(b), wd, shd, flags=moe.F_ACCUMULATE, out=resid)
    torch.cuda.synchronize()
    acc_ref = ref["out"] + host(r1["out"])
    assert_close(host(r3["out"]), acc_ref, what="accumulate")


def test_layer_forward_k_equal_E_identical_experts():
    """Test (ii) on the GPU: k = E with all experts equal reduces to one dense FFN."""
    s = mi.LayerSpec("ident", 12, 128, 64, 8, 8, 0, 0, "bf16", "bf16", 1.0, 0.05, 0.05, seed=9)
    x = mi.host_x(s)
    wr, b = mi.host_router(s)
    w = mi.host_experts(s, experts=[0] * s.E)
    ref = oracle.layer_forward(s, x, wr, b, w)
    res = moe.layer_forward(s, dev(x), dev(wr), dev(b), {k: dev(v) for k, v in w.items()})
    torch.cuda.synchronize()
    assert_close(host(res["out"]), ref["out"], what="k=E identical experts")
    assert sorted(host(res["topk_idx"])[0].tolist()) == list(range(8))


def test_layer_forward_skewed_routing_and_empty_batch():
    """Every token routed to the same experts (huge bias); and T = 0 is a no-op."""
    s = mi.LayerSpec("skew", 24, 256, 64, 16, 2, 1, 64, "bf16", "bf16", 1.0, 0.05, 0.05, seed=10)
    x = mi.host_x(s)
    wr, _ = mi.host_router(s)
    b = np.zeros(s.E, np.float32)
    b[[3, 11]] = 1000.0
    w, sh, wd, shd = _weights(s)
    ref = oracle.layer_forward(s, x, wr, b, w, sh)
    assert set(ref["topk_idx"].reshape(-1).tolist()) == {3, 11}
    res = moe.layer_forward(s, dev(x), dev(wr), dev(b), wd, shd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(res["topk_idx"]), ref["topk_idx"])
    assert_close(host(res["out"]), ref["out"], what="skewed")
    shape = moe.make_shape(s, T=0)
    out = torch.empty((1, s.d), dtype=torch.bfloat16, device="cuda")
    moe.layer_forward_raw(shape, dev(x), dev(wr), dev(b), moe.make_weights(wd, shd), out)


DECODE_ODD = [
    mi.LayerSpec("dec_fs_gt_f", 7, 256, 64, 16, 3, 1, 192, "bf16", "bf16", 1.0, 0.05, 0.05, seed=31),
    mi.LayerSpec("dec_fs_lt_f", 5, 256, 192, 16, 3, 1, 64, "bf16", "bf16", 1.0, 0.05, 0.05, seed=32),
    mi.LayerSpec("dec_mxfp4_shared", 3, 128, 96, 12, 4, 1, 64, "bf16", "mxfp4", 1.0, 0.0, 0.05, seed=33),
    mi.LayerSpec("dec_long_k", 2, 4096, 64, 8, 2, 1, 32, "bf16", "bf16", 1.0, 0.02, 0.02, seed=34),
    mi.LayerSpec("dec_long_f", 3, 64, 2048, 8, 2, 0, 0, "bf16", "bf16", 1.0, 0.02, 0.02, seed=35),
    mi.LayerSpec("dec_f32_E1", 4, 64, 32, 1, 1, 0, 0, "f32", "f32", 0.5, 0.1, 0.1, seed=36),
    # a single token: the down kernel that splits (slot, row) units over the wavefronts
    mi.LayerSpec("dec1_fs_gt_f", 1, 256, 64, 16, 3, 1, 192, "bf16", "bf16", 1.0, 0.05, 0.05, seed=37),
    mi.LayerSpec("dec1_fs_lt_f", 1, 256, 192, 16, 9, 1, 64, "bf16", "bf16", 1.0, 0.05, 0.05, seed=38),
    mi.LayerSpec("dec1_mxfp4_k12", 1, 160, 96, 24, 12, 1, 64, "bf16", "mxfp4", 1.0, 0.0, 0.05, seed=39),
    mi.LayerSpec("dec1_f32", 1, 100, 40, 8, 5, 1, 24, "f32", "f32", 0.5, 0.1, 0.1, seed=40),
    mi.LayerSpec("dec1_long_f", 1, 64, 2048, 8, 2, 0, 0, "bf16", "bf16", 1.0, 0.02, 0.02, seed=41),
    # a single token the per-wavefront gate/up routing leaves to the general one: rows longer than
    # one K step, and more than 256 experts
    mi.LayerSpec("dec1_long_k", 1, 4096, 64, 8, 2, 1, 32, "bf16", "bf16", 1.0, 0.02, 0.02, seed=42),
    mi.LayerSpec("dec1_E300", 1, 128, 64, 300, 4, 0, 0, "bf16", "bf16", 1.0, 0.05, 0.05, seed=43),
]


@pytest.mark.parametrize("s", DECODE_ODD, ids=lambda s: s.name)
def test_layer_forward_decode_odd_shapes(s):
    """Shared d_ff larger / smaller than the routed one, rows longer than one K step, E = 1."""
    x, wr, b, _ = margin_x(s)
    w, sh, wd, shd = _weights(s)
    ref = oracle.layer_forward(s, x, wr, b, w, sh)
    res = moe.layer_forward(s, dev(x), dev(wr), dev(b), wd, shd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(res["topk_idx"]), ref["topk_idx"])
    assert_close(host(res["out"]), ref["out"], what=s.name)


@pytest.mark.parametrize("T", [1, 3])
def test_stack_forward_small(T):
    """moe_stack_forward over 3 layers against the oracle's stack layer applied 3 times."""
    s = mi.LayerSpec("stk", T, 256, 128, 16, 3, 0, 0, "bf16", "mxfp4", 1.0, 0.0, 0.05, seed=41, n_layers=3)
    rng = np.random.default_rng(5)
    h0 = rng.normal(size=(T, s.d)).astype(np.float32)
    layers = [(mi.host_router(s, l), mi.host_experts(s, l)) for l in range(3)]
    h_ref = h0.copy()
    idx_ref = [oracle.stack_layer(s, h_ref, wr, b, w) for (wr, b), w in layers]
    shape = moe.make_shape(s)
    h = dev(h0)
    wds = [{k: dev(v) for k, v in w.items()} for _, w in layers]
    moe.stack_forward(shape, h, [dev(wr) for (wr, _), _ in layers], [dev(b) for (_, b), _ in layers],
                      [moe.make_weights(wd) for wd in wds])
    torch.cuda.synchronize()
    assert_close(host(h), h_ref.astype(np.float64), what=f"stack T={T}")


@pytest.mark.parametrize("T", [1, 4])
def test_stack_graph_replays_match_eager(T):
    """The stack captured once in a HIP graph (as the benchmark times the 43-layer stack):
    three replays on fresh inputs, with eager library calls and synchronisations between them,
    each equal bit for bit to an eager call on the same input."""
    s = mi.LayerSpec("stkg", T, 256, 128, 16, 3, 0, 0, "bf16", "mxfp4", 1.0, 0.0, 0.05, seed=43, n_layers=3)
    rng = np.random.default_rng(9)
    wrs, bs, Ws, keep = [], [], [], []
    for l in range(3):
        wr, b = mi.host_router(s, l)
        wd = {k: dev(v) for k, v in mi.host_experts(s, l).items()}
        wrs.append(dev(wr))
        bs.append(dev(b))
        Ws.append(moe.make_weights(wd))
        keep.append(wd)
    shape = moe.make_shape(s)
    ws = moe.workspace(shape)
    inputs = [dev(rng.normal(size=(T, s.d)).astype(np.float32)) for _ in range(3)]
    h = torch.empty((T, s.d), dtype=torch.float32, device="cuda")
    refs = []
    for x in inputs:
        h.copy_(x)
        moe.stack_forward(shape, h, wrs, bs, Ws, ws)
        refs.append(h.clone())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    h.copy_(inputs[0])
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        moe.stack_forward(shape, h, wrs, bs, Ws, ws)
    other = torch.empty_like(h)
    for i, x in enumerate(inputs):
        h.copy_(x)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(h, refs[i]), f"replay {i} differs from the eager stack"
        other.copy_(inputs[(i + 1) % 3])  # eager work between replays
        moe.stack_forward(shape, other, wrs, bs, Ws, ws)
        torch.cuda.synchronize()
        assert torch.equal(other, refs[(i + 1) % 3])


def test_no_renorm_gates():
    s = mi.spec("c1", T=16)
    x, wr, b, _ = margin_x(s)
    l32, _ = oracle.router_logits(s, x, wr, b)
    ref_idx, ref_w = oracle.topk(s, l32, flags=oracle.NO_RENORM)
    shape = moe.make_shape(s, flags=moe.F_NO_RENORM)
    idx = torch.empty((16, s.k), dtype=torch.int32, device="cuda")
    w = torch.empty((16, s.k), dtype=torch.float32, device="cuda")
    moe.route(shape, dev(x), dev(wr), dev(b), idx, w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(idx), ref_idx)
    np.testing.assert_allclose(host(w), ref_w, rtol=2e-5, atol=1e-8)


@pytest.mark.parametrize("E,k,tied,T", [(16, 4, [1, 3, 6, 10, 12], 3), (256, 6, [3, 7, 100, 101, 200, 201, 255], 1),
                                        (128, 8, [0, 5, 9, 64, 65, 127, 100, 99, 98], 2), (64, 2, [63, 0, 31], 5)])
def test_decode_routing_exact_ties(E, k, tied, T):
    """Equal router rows give bit-equal logits; the decode layer keeps the lower expert index among
    equal logits, also when the tie straddles the k-th place, and lists equal logits by index."""
    s = mi.LayerSpec("ties", T, 128, 64, E, k, 0, 0, "bf16", "bf16", 1.0, 0.05, 0.05, seed=50)
    x = mi.host_x(s)
    wr, _ = mi.host_router(s)
    wr = wr.copy()
    wr[tied] = wr[tied[0]]
    b = np.zeros(E, np.float32)
    b[tied] = 50.0
    w = mi.host_experts(s)
    ref = oracle.layer_forward(s, x, wr, b, w)
    assert (ref["topk_idx"] == np.array(sorted(tied)[:k])).all()
    res = moe.layer_forward(s, dev(x), dev(wr), dev(b), {n: dev(v) for n, v in w.items()})
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(res["topk_idx"]), ref["topk_idx"])
    assert_close(host(res["out"]), ref["out"], what="ties")


@pytest.mark.parametrize("T", [1, 3])
def test_decode_routing_signed_zero_inf_nan(T):
    """Decode routing order on special logits: +0 and -0 tie (lower index first), -inf ranks below
    every finite logit and NaN below -inf (so with k = 6 of 8 the NaN experts stay out)."""
    E, k = 8, 6
    s = mi.LayerSpec("specials", T, 128, 64, E, k, 0, 0, "bf16", "bf16", 1.0, 0.05, 0.05, seed=51)
    x = mi.host_x(s)
    wr, _ = mi.host_router(s)
    wr = wr.copy()
    special = [1, 2, 3, 4, 5, 7]
    wr[special] = 0.0   # these experts' logits are their bias exactly
    b = np.full(E, -1.0e4, np.float32)
    b[[1, 7]] = np.nan
    b[2], b[3], b[4], b[5] = -0.0, -np.inf, 0.0, 1.0
    w = mi.host_experts(s)
    ref = oracle.layer_forward(s, x, wr, b, w)
    assert (ref["topk_idx"][:, :3] == [5, 2, 4]).all() and (ref["topk_idx"][:, 5] == 3).all()
    res = moe.layer_forward(s, dev(x), dev(wr), dev(b), {n: dev(v) for n, v in w.items()})
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(res["topk_idx"]), ref["topk_idx"])
    assert_close(host(res["out"]), ref["out"], what="specials")


@pytest.mark.parametrize("s", [mi.spec("c1", T=4), mi.spec("c3", T=1),
                               mi.LayerSpec("ws_gemm", 333, 256, 128, 16, 4, 1, 192, "bf16", "bf16", 1.0, 0.05, 0.05,
                                            seed=21)], ids=lambda s: f"{s.name}_T{s.T}")
def test_workspace_needs_no_initialisation(s):
    """The same layer through a workspace full of 0xFF bytes and through a zeroed one: bit-equal
    outputs and routing (no kernel reads a workspace region before writing it)."""
    x, wr, b, _ = margin_x(s)
    w, sh, wd, shd = _weights(s)
    shape = moe.make_shape(s)
    W = moe.make_weights(wd, shd)
    n = moe.workspace_size(shape)
    outs = []
    for fill in (0x00, 0xFF):
        ws = torch.full((n,), fill, dtype=torch.uint8, device="cuda")
        out = torch.empty((s.T, s.d), dtype=torch.bfloat16, device="cuda")
        idx = torch.empty((s.T, s.k), dtype=torch.int32, device="cuda")
        moe.layer_forward_raw(shape, dev(x), dev(wr), dev(b), W, out, idx, ws)
        torch.cuda.synchronize()
        outs.append((out, idx))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    ref = oracle.layer_forward(s, x, wr, b, w, sh)
    np.testing.assert_array_equal(host(outs[1][1]), ref["topk_idx"])
    assert_close(host(outs[1][0]), ref["out"], what=f"{s.name} T={s.T} through a 0xFF workspace")
