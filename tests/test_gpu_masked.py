"""GPU parity of the partial layer (moe_layer_forward_masked).

The combine restricted to a subset of the experts, and the exact merge of complementary partial
layers: a partial layer over experts A, then one over the rest with MOE_F_ACCUMULATE, gives the
full layer (the merge of the GPU's and the CPU's partial sums in the pages' scheduler:
dothoosh.com FreeToken article, "FreeToken architecture and the sparsity puzzle", mechanism 1).
Covers the decode path (bf16 + shared, MXFP4, fp32), the grouped-GEMM path and the grouped-GEMV
path, against the oracle's masked layer.
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

CASES = [
    mi.spec("c1", T=1),                # decode, bf16 + shared
    mi.spec("c1", T=16),
    mi.spec("c3", T=8),                # decode, MXFP4
    mi.spec("c0"),                     # decode, fp32
    mi.spec("c0", T=48),               # grouped GEMV path (fp32, T > 32)
    mi.LayerSpec("g_bf16", 333, 256, 128, 16, 4, 1, 192, "bf16", "bf16", 1.0, 0.05, 0.05, seed=21),       # GEMM
    mi.LayerSpec("g_mxfp4_shared", 64, 256, 128, 8, 8, 1, 128, "bf16", "mxfp4", 1.0, 0.0, 0.05, seed=24),  # GEMM
]


def _torch_dtype(s):
    return torch.float32 if s.act == "f32" else torch.bfloat16


@pytest.mark.parametrize("s", CASES, ids=lambda s: f"{s.name}_T{s.T}")
def test_partial_layers_match_oracle_and_merge(s):
    x, wr, b, _ = margin_x(s)
    w = mi.host_experts(s)
    sh = mi.host_experts(s, shared=True) if s.n_shared else None
    wd = {k: dev(v) for k, v in w.items()}
    shd = {k: dev(v) for k, v in sh.items()} if sh is not None else None
    W = moe.make_weights(wd, shd)
    full_ref = oracle.layer_forward(s, x, wr, b, w, sh)
    rng = np.random.default_rng(s.seed + 7)
    for trial in range(2):
        mask_a = (rng.random(s.E + 1) < 0.5).astype(np.uint8)
        mask_b = (1 - mask_a).astype(np.uint8)
        ref_a = oracle.layer_forward(s, x, wr, b, w, sh, expert_mask=mask_a)["out"]
        out = torch.empty((s.T, s.d), dtype=_torch_dtype(s), device="cuda")
        idx = torch.empty((s.T, s.k), dtype=torch.int32, device="cuda")
        moe.layer_forward_masked_raw(moe.make_shape(s), dev(x), dev(wr), dev(b), W, dev(mask_a), out, idx)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(idx), full_ref["topk_idx"])
        assert_close(host(out), ref_a, what=f"{s.name} partial A (trial {trial})")
        moe.layer_forward_masked_raw(moe.make_shape(s, flags=moe.F_ACCUMULATE), dev(x), dev(wr), dev(b), W,
                                     dev(mask_b), out)
        torch.cuda.synchronize()
        assert_close(host(out), full_ref["out"], what=f"{s.name} A + B merged (trial {trial})")


@pytest.mark.parametrize("s", [mi.spec("c1", T=4), CASES[5]], ids=lambda s: f"{s.name}_T{s.T}")
def test_empty_mask_computes_nothing(s):
    """No expert in the mask: the output is zero, and with MOE_F_ACCUMULATE it is left as it was."""
    x, wr, b, _ = margin_x(s)
    w = mi.host_experts(s)
    sh = mi.host_experts(s, shared=True) if s.n_shared else None
    W = moe.make_weights({k: dev(v) for k, v in w.items()}, {k: dev(v) for k, v in sh.items()} if sh else None)
    zero = torch.zeros(s.E + 1, dtype=torch.uint8, device="cuda")
    out = torch.full((s.T, s.d), 3.0, dtype=_torch_dtype(s), device="cuda")
    moe.layer_forward_masked_raw(moe.make_shape(s, flags=moe.F_ACCUMULATE), dev(x), dev(wr), dev(b), W, zero, out)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
    moe.layer_forward_masked_raw(moe.make_shape(s), dev(x), dev(wr), dev(b), W, zero, out)
    torch.cuda.synchronize()
    assert torch.all(out == 0.0)
