"""GPU parity of the NVFP4 weight path (E2M1 codes, one FP8 E4M3 scale per 16 elements, one
fp32 scale per tensor: the 4-bit build named in the aihot.vn FreeToken article, "Flags", and
the dothoosh.com FreeToken article, "Editorial"; the layout is NVIDIA's published one).

- moe_nvfp4_dequant: every code x every scale byte x three tensor scales, bit for bit.
- The whole layer through the decode kernels (T <= 32) and the grouped-GEMV kernels (T > 32),
  routed-only at the DeepSeek-V4-Flash layer size and small shapes with a shared expert,
  against the oracle's NVFP4 layer, to the layer's floating tolerance.
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


def _dev_weights(w):
    return {k: (dev(v) if isinstance(v, np.ndarray) else v) for k, v in w.items()}


@pytest.mark.parametrize("gscale", [1.0, 0.3, 3.0e-39])
def test_nvfp4_dequant_table_bit_exact(gscale):
    # each row: the 16 codes twice (32 elements), scale byte i on its first half and
    # (5 i + 3) mod 256 on its second, so all 256 bytes meet every code in both halves
    codes = np.array(list(range(16)) * 2, np.uint8)
    packed = np.tile((codes[0::2] | (codes[1::2] << 4)).astype(np.uint8), (256, 1))
    i = np.arange(256)
    scales = np.stack([i, (5 * i + 3) % 256], axis=1).astype(np.uint8)
    ref = oracle.nvfp4_dequant(packed, scales, gscale)
    out = torch.empty((256, 32), dtype=torch.float32, device="cuda")
    moe.nvfp4_dequant(dev(packed), dev(scales), gscale, out)
    torch.cuda.synchronize()
    got = host(out)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    bad = np.nonzero((got.view(np.uint32) != ref.view(np.uint32)) & ~nan)
    assert bad[0].size == 0, f"mismatch at rows {sorted(set(bad[0].tolist()))[:20]}"


def test_nvfp4_dequant_many_rows():
    rng = np.random.default_rng(5)
    rows, K = 777, 96
    packed = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, (rows, K // 16), dtype=np.uint8)
    ref = oracle.nvfp4_dequant(packed, scales, 0.6)
    out = torch.empty((rows, K), dtype=torch.float32, device="cuda")
    moe.nvfp4_dequant(dev(packed), dev(scales), 0.6, out)
    torch.cuda.synchronize()
    got = host(out)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got.view(np.uint32)[~nan], ref.view(np.uint32)[~nan])


SMALL = [
    mi.LayerSpec("nv_shared", 3, 128, 96, 12, 4, 1, 64, "bf16", "nvfp4", 1.0, 0.0, 0.05, scale_lo=0x20,
                 scale_hi=0x3F, seed=41),
    mi.LayerSpec("nv_fs_gt_f", 9, 256, 64, 16, 3, 1, 192, "bf16", "nvfp4", 1.0, 0.0, 0.05, scale_lo=0x20,
                 scale_hi=0x3F, seed=42),
    mi.LayerSpec("nv_gemv", 48, 256, 128, 16, 4, 1, 96, "bf16", "nvfp4", 1.0, 0.0, 0.05, scale_lo=0x20,
                 scale_hi=0x3F, seed=43),     # T > 32: grouped-GEMV kernels
    mi.LayerSpec("nv_gemv_ragged", 77, 160, 224, 8, 2, 0, 0, "bf16", "nvfp4", 1.0, 0.0, 0.05, scale_lo=0x20,
                 scale_hi=0x3F, seed=44),
]


def _layer_case(s):
    x, wr, b, _ = margin_x(s)
    w = mi.host_experts(s)
    sh = mi.host_experts(s, shared=True) if s.n_shared else None
    ref = oracle.layer_forward(s, x, wr, b, w, sh)
    res = moe.layer_forward(s, dev(x), dev(wr), dev(b), _dev_weights(w), _dev_weights(sh) if sh else None)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(res["topk_idx"]), ref["topk_idx"])
    assert_close(host(res["out"]), ref["out"], what=f"{s.name} T={s.T} out")
    return w, sh, x, wr, b, ref


@pytest.mark.parametrize("s", SMALL, ids=lambda s: s.name)
def test_nvfp4_layer_small(s):
    _layer_case(s)


@pytest.mark.parametrize("T", [1, 8, 32])
def test_nvfp4_layer_full_size_decode(T):
    """E = 256, k = 6, d = 4096, f = 2048: the DeepSeek-V4-Flash routed layer, NVFP4 weights."""
    _layer_case(mi.spec("c3nv", T=T))


def test_nvfp4_gemv_path_matches_decode_path():
    """The same batch through the decode kernels and, forced, through the grouped-GEMV kernels."""
    s = SMALL[1]
    x, wr, b, _ = margin_x(s)
    w, sh = mi.host_experts(s), mi.host_experts(s, shared=True)
    ref = oracle.layer_forward(s, x, wr, b, w, sh)
    wd, shd = _dev_weights(w), _dev_weights(sh)
    r1 = moe.layer_forward(s, dev(x), dev(wr), dev(b), wd, shd)
    r2 = moe.layer_forward(s, dev(x), dev(wr), dev(b), wd, shd, flags=moe.F_FORCE_GEMV)
    torch.cuda.synchronize()
    assert_close(host(r1["out"]), ref["out"], what="decode path")
    assert_close(host(r2["out"]), ref["out"], what="grouped-GEMV path")


def test_nvfp4_tensor_scale_is_applied():
    """Halving both routed tensor scales halves the routed contribution (E4M3 x E2M1 products
    are exact, so the decoded weights scale exactly); the oracle agrees."""
    s = SMALL[3].with_T(5)
    x, wr, b, _ = margin_x(s)
    w = mi.host_experts(s)
    w_half = dict(w, w13_gscale=w["w13_gscale"] / 2, w2_gscale=w["w2_gscale"] / 2)
    ref = oracle.layer_forward(s, x, wr, b, w_half)
    res = moe.layer_forward(s, dev(x), dev(wr), dev(b), _dev_weights(w_half))
    torch.cuda.synchronize()
    assert_close(host(res["out"]), ref["out"], what="half tensor scales")
