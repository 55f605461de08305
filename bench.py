"""Benchmark of the routed MoE layer on one MI355X through the C-ABI library.

A step is one pass of the whole layer (router logits, top-k + gates, permute, grouped
expert FFNs, combine; for the stack, 43 such layers with the RMS-norm residual glue)
over one batch of synthetic tokens already resident in HBM.  The headline workload is the
largest single-GPU configuration, the 43-layer MXFP4 stack of the 256-expert top-6 layer
decoding one token (all 147 GB of expert weights resident); every other workload runs as a
sweep entry with the same fields (roofline object, CPU baseline) in the same JSON line.

Decode steps draw a fresh token batch from a pool of 256 batches and rotate through
several copies of the layer's weights (like successive layers of a model), so the
256 MB Infinity Cache cannot serve repeated weight reads.

Timing: hipEvents on the stream the library launches on (torch's current stream).
Pass 1 times K steps end to end (value, ms_per_step), with events between five consecutive
groups of the steps for the median of five repeats (ms_per_step_median_of_5).  Pass 2 repeats K steps with the
library's timing hook bracketing the gate/up FFN kernel (the largest share of the
layer's bytes and flops) to get that kernel's average duration for the roofline; pass 3
does the same for the down projection.  The device's own peaks (an HBM read stream, the
bf16 and fp8 x fp4 matrix instructions) are measured once and every fraction is also
reported against them.

The CPU baseline is the oracle as it stands (plain C, fp64 sums, OpenMP over output
elements) on a bounded sample of each workload's tokens, timed on the host's cores; for
the 43-layer stack it is three sampled layers (0, 21, 42), scaled by 43.  The oracle's
single-threaded rates on the tiny, bf16 decode and MXFP4 decode layers come from child
processes with one OpenMP thread.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-sweep]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
FP8_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 MFMA, published (the fp8 x fp4 scaled MFMA runs at the fp8 rate)

WORKLOADS = {
    # name: (config, T, weight copies, description)
    "c1_decode_T1": ("c1", 1, 8, "decode, bf16, E=128 top-8 + 1 shared, d=2048, f=768, T=1"),
    "c1_decode_T4": ("c1", 4, 8, "decode, bf16, E=128 top-8 + 1 shared, d=2048, f=768, T=4"),
    "c1_decode_T16": ("c1", 16, 8, "decode, bf16, E=128 top-8 + 1 shared, d=2048, f=768, T=16"),
    "c2_prefill": ("c2", 4096, 1, "prefill, bf16, E=128 top-8 + 1 shared, d=2048, f=768, T=4096"),
    "c2_skew_prefill": ("c2_skew", 4096, 1, "prefill, bf16, Zipf(1.1) router prior, T=4096"),
    "c3_decode_T1": ("c3", 1, 4, "decode, MXFP4 weights, E=256 top-6, d=4096, f=2048, T=1"),
    "c3_decode_T8": ("c3", 8, 4, "decode, MXFP4 weights, E=256 top-6, d=4096, f=2048, T=8"),
    "c3_decode_T32": ("c3", 32, 4, "decode, MXFP4 weights, E=256 top-6, d=4096, f=2048, T=32"),
    "c3_prefill": ("c3", 8192, 1, "prefill, MXFP4 weights, E=256 top-6, d=4096, f=2048, T=8192"),
    "c3_prefill_mx": ("c3", 8192, 1, "prefill, MXFP4 weights on the fp8 x fp4 matrix cores, activations quantised to "
                                     "MXFP8 (MOE_F_MX_GEMM), E=256 top-6, d=4096, f=2048, T=8192"),
    "c3nv_decode_T1": ("c3nv", 1, 4, "decode, NVFP4 weights, E=256 top-6, d=4096, f=2048, T=1"),
    "c3nv_decode_T8": ("c3nv", 8, 4, "decode, NVFP4 weights, E=256 top-6, d=4096, f=2048, T=8"),
    "c4_stack": ("c4", 1, 1, "43-layer MXFP4 stack of the E=256 top-6 layer, T=1, RMS-norm residual"),
    "c4_stack_persistent": ("c4", 1, 1, "43-layer MXFP4 stack of the E=256 top-6 layer, T=1, RMS-norm residual, "
                                        "one persistent cooperative launch (grid barriers between the steps)"),
}
# the tiny fp32 layer is a parity case, not a GPU workload; the oracle's single-threaded rate on it
# is reported beside the others
CPU_ONLY = {"c0_tiny_T16": ("c0", 16, 1, "tiny fp32 layer, E=8 top-2, d=256, f=128, T=16")}
HEADLINE = "c4_stack"
MX_WORKLOADS = {"c3_prefill_mx"}  # run with MOE_F_MX_GEMM
POOL = 256

# HBM traffic of the roofline kernel, from two rocprofv3 --pmc passes (FETCH_SIZE, then
# WRITE_SIZE, KiB per dispatch, averaged over the dispatches of the bench command) scaled by
# what the same counters read for a plain device-to-device copy of 256 MiB.  Each entry names
# the digest of the kernel sources it was taken on; a different digest reports null.
KERNEL_SOURCES = {
    "decode": ["decode.hip", "common.h", "wchunk.h"],
    "gemm": ["gemm.hip", "common.h", "wchunk.h", "lds_dma.h", "mxfp8.h"],
    "mx": ["mxgemm.hip", "common.h", "lds_dma.h", "mxfp8.h"],
}
COPY_CAL = dict(fetch_factor=1.99981, write_factor=1.00000)  # profiles/read_counters__calibration.txt
TRAFFIC = {  # workload -> counters of its roofline kernel (profiles/<kernel>__<workload>.txt)
    "c1_decode_T1": dict(src="decode:ffe63db048e10eda", fetch_kib=27747.6, write_kib=54.3),
    "c3_decode_T1": dict(src="decode:ffe63db048e10eda", fetch_kib=26241.9, write_kib=96.3),
    "c3nv_decode_T1": dict(src="decode:ffe63db048e10eda", fetch_kib=27761.8, write_kib=96.2),
    "c4_stack": dict(src="decode:ffe63db048e10eda", fetch_kib=26241.8, write_kib=96.3),
    "c4_stack_persistent": dict(src="decode:ffe63db048e10eda", fetch_kib=1751435.4, write_kib=20210.0),
    "c2_prefill": dict(src="gemm:9b7c98358210386a", fetch_kib=550290.0, write_kib=110649.8),
    "c3_prefill": dict(src="gemm:9b7c98358210386a", fetch_kib=1860059.2, write_kib=298145.2),
    "c3_prefill_mx": dict(src="mx:17c5a4a5b4bc3658", fetch_kib=1383077.5, write_kib=102177.9),
}


def _code_only(src: str) -> str:
    """C/HIP source without comments, whitespace runs collapsed (string literals kept as is)."""
    import re
    tok = re.compile(r'"(?:\\.|[^"\\])*"|\'(?:\\.|[^\'\\])*\'|//[^\n]*|/\*.*?\*/', re.S)
    body = tok.sub(lambda m: " " if m.group(0)[0] == "/" else m.group(0), src)
    return " ".join(body.split())


def source_digest(kind: str) -> str:
    """Digest of the code (comments and layout excluded) of one kernel family's sources."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "sparse_mixture_experts_16_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return f"{kind}:{h.hexdigest()[:16]}"


def traffic_bytes(workload: str):
    t = TRAFFIC.get(workload)
    if not t or not COPY_CAL or t["src"] != source_digest(t["src"].split(":")[0]):
        return None
    return t["fetch_kib"] * 1024 * COPY_CAL["fetch_factor"] + t["write_kib"] * 1024 * COPY_CAL["write_factor"]


def copy_calibration():
    """The counters' references: a plain 256 MiB device-to-device copy, 5 times; then 5 reads each
    of the same 256 MiB by the whole-line stream (peak_hbm_read) and in the prefill GEMM's
    tile-row pattern (64-byte pieces of 4096-byte rows), through registers and through LDS."""
    import torch
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_mixture_experts_16_amd", "libmoe_peaks.so"))
    lib.peak_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.peak_rows64_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    out = torch.empty(n // 256, dtype=torch.int32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for _ in range(5):
        assert lib.peak_hbm_read(a.data_ptr(), n, 2048, out.data_ptr(), st) == 0
    for dma in (0, 1):
        for _ in range(5):
            assert lib.peak_rows64_read(a.data_ptr(), n, dma, out.data_ptr(), st) == 0
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "read_bytes_per_launch": n, "launches": 5}))


def expert_bytes(s, f=None):
    """Bytes of one expert's weights (w13 + w2), split (up, down)."""
    f = s.f if f is None else f
    if s.wt in ("mxfp4", "nvfp4"):
        blk = 32 if s.wt == "mxfp4" else 16  # elements per scale byte
        up = 2 * f * s.d // 2 + 2 * f * s.d // blk
        down = s.d * f // 2 + s.d * f // blk
    else:
        eb = 4 if s.wt == "f32" else 2
        up, down = 2 * f * s.d * eb, s.d * f * eb
    return up, down


class Hip:
    """hipEvent_t plumbing through the HIP runtime torch already loaded."""

    def __init__(self):
        import torch  # noqa: F401
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        rc = self.lib.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return e.value

    def record(self, ev, stream):
        rc = self.lib.hipEventRecord(ev, stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, a, b):
        self.lib.hipEventSynchronize(b)
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def destroy(self, ev):
        self.lib.hipEventDestroy(ev)


REPEATS = 5  # the timed steps are split into this many consecutive groups for the median


def _timed(hip, stream, step, steps, warmup, profile=None):
    """Run warmup + timed steps.  Unprofiled: (total ms, ms per step of each of REPEATS
    consecutive groups of the steps, events between groups).  Profiled: (None, per-step ms of
    the profiled kernel)."""
    import torch
    import sparse_mixture_experts_16_amd as moe
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    kern = []
    if profile is None:
        cuts = sorted({steps * g // REPEATS for g in range(REPEATS + 1)})
        evs = [hip.event() for _ in cuts]
        hip.record(evs[0], stream)
        for i in range(steps):
            step(warmup + i)
            if i + 1 in cuts:
                hip.record(evs[cuts.index(i + 1)], stream)
        torch.cuda.synchronize()
        total = hip.elapsed_ms(evs[0], evs[-1])
        groups = [hip.elapsed_ms(evs[g], evs[g + 1]) / (cuts[g + 1] - cuts[g]) for g in range(len(cuts) - 1)]
        for e in evs:
            hip.destroy(e)
        return total, groups
    evs = [(hip.event(), hip.event()) for _ in range(steps)]
    for i in range(steps):
        moe.profile_kernel(profile, evs[i][0], evs[i][1])
        step(warmup + i)
    moe.profile_kernel(-1)
    torch.cuda.synchronize()
    for a, b in evs:
        try:
            kern.append(hip.elapsed_ms(a, b))
        except RuntimeError:  # no launch of that kernel class in the step
            hip.lib.hipGetLastError()  # clear the failed query's error
        hip.destroy(a)
        hip.destroy(b)
    return None, kern


def run_layer_workload(hip, name, steps, warmup):
    import torch
    import moe_inputs as mi
    import sparse_mixture_experts_16_amd as moe
    cfg, T, copies, desc = WORKLOADS[name]
    s = mi.spec(cfg, T=T)
    decode = T <= 32
    n_batches = POOL if decode else 2
    stream = torch.cuda.current_stream().cuda_stream
    # Inputs: a pool of token batches (distinct token rows), weight copies, router per copy.
    x_all = mi.host_x(mi.spec(cfg, T=T * n_batches))
    x_pool = _to_dev(x_all).reshape(n_batches, T, s.d)
    layers = []
    for c in range(copies):
        wr, b = mi.host_router(s, layer=c)
        w = mi.device_experts(s, layer=c)
        sh = mi.device_experts(s, layer=c, shared=True) if s.n_shared else None
        layers.append((_to_dev(wr), _to_dev(b), moe.make_weights(w, sh), w, sh))
    mx = name in MX_WORKLOADS
    shape = moe.make_shape(s, flags=moe.F_MX_GEMM if mx else 0)
    ws = moe.workspace(shape)
    out = torch.empty((T, s.d), dtype=torch.bfloat16, device="cuda")
    row = (T * s.k + 3) // 4 * 4  # keep every step's slice 16-byte aligned
    idx_log = torch.empty((max(steps, 1), row), dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()

    def step(i, log=None):
        wr, b, W, _, _ = layers[i % copies]
        moe.layer_forward_raw(shape, x_pool[i % n_batches], wr, b, W, out,
                              idx_log[log, :T * s.k] if log is not None else None, ws)

    total, groups = _timed(hip, stream, step, steps, warmup)
    _, k_up = _timed(hip, stream, lambda i: step(i, log=(i - warmup) if i >= warmup else None), steps, warmup,
                     profile=moe.KERNEL_FFN_UP)
    _, k_down = _timed(hip, stream, step, steps, warmup, profile=moe.KERNEL_FFN_DOWN)
    torch.cuda.synchronize()
    # Routing actually taken (timed pass 2 logged it) -> unique experts per step.
    idx = idx_log[:, :T * s.k].cpu().numpy()
    uniq = np.array([len(np.unique(idx[i])) for i in range(steps)], np.float64)
    counts = np.bincount(idx.reshape(-1), minlength=s.E)
    up_b, down_b = expert_bytes(s)
    sh_up, sh_down = expert_bytes(s, s.f_shared) if s.n_shared else (0, 0)
    ms = total / steps
    rec = dict(workload=name, desc=desc, T=T, ms_per_step=ms, tokens_per_s=T / (ms * 1e-3),
               ms_per_step_median_of_5=float(np.median(groups)),
               ffn_up_us=float(np.mean(k_up) * 1e3), ffn_down_us=float(np.mean(k_down) * 1e3) if k_down else None,
               experts_hit_per_step=float(uniq.mean()),
               experts_never_hit=int((counts == 0).sum()), load_max_over_mean=float(counts.max() / counts.mean()))
    if decode:
        layer_bytes = uniq * (up_b + down_b) + s.n_shared * (sh_up + sh_down)
        up_bytes = uniq * up_b + s.n_shared * sh_up
        rec["bound"] = "hbm"
        rec["alg_bytes_per_step"] = float(layer_bytes.mean())
        rec["step_GBps"] = float(layer_bytes.mean() / (ms * 1e-3) / 1e9)
        rec["step_frac_hbm"] = rec["step_GBps"] / HBM_PEAK_GBS
        rec["ffn_up_alg_bytes"] = float(up_bytes.mean())
        rec["ffn_up_GBps"] = float(np.mean(up_bytes / (np.array(k_up) * 1e-3)) / 1e9)
        rec["ffn_up_frac"] = rec["ffn_up_GBps"] / HBM_PEAK_GBS
    else:
        rows = T * s.k + s.n_shared * T
        fl_up = 2.0 * rows * 2 * s.f * s.d
        fl_layer = 3.0 / 2.0 * fl_up + 2.0 * T * s.E * s.d
        peak = FP8_PEAK_TFLOPS if mx else BF16_PEAK_TFLOPS
        rec["bound"] = "mfma"
        rec["mfma_dtype"] = "fp8 x fp4 (scaled)" if mx else "bf16"
        rec["alg_flops_per_step"] = fl_layer
        rec["step_TFLOPs"] = fl_layer / (ms * 1e-3) / 1e12
        rec["step_frac_mfma"] = rec["step_TFLOPs"] / peak
        rec["ffn_up_alg_flops"] = fl_up
        rec["ffn_up_TFLOPs"] = fl_up / (np.mean(k_up) * 1e-3) / 1e12
        rec["ffn_up_frac"] = rec["ffn_up_TFLOPs"] / peak
    del layers, x_pool, ws, out, idx_log
    moe._ws_cache.clear()
    torch.cuda.empty_cache()
    return rec


def run_stack_workload(hip, steps, warmup, persistent=False):
    import torch
    import moe_inputs as mi
    import sparse_mixture_experts_16_amd as moe
    s = mi.spec("c4")
    stream = torch.cuda.current_stream().cuda_stream
    wrs, bs, Ws, keep = [], [], [], []
    for l in range(s.n_layers):
        wr, b = mi.host_router(s, layer=l)
        w = mi.device_experts(s, layer=l)
        wrs.append(_to_dev(wr))
        bs.append(_to_dev(b))
        Ws.append(moe.make_weights(w))
        keep.append(w)
    h0 = _to_dev(mi.host_h0(mi.spec("c4", T=POOL)))
    h = torch.empty((1, s.d), dtype=torch.float32, device="cuda")
    shape = moe.make_shape(s)
    ws = moe.workspace(shape)
    torch.cuda.synchronize()

    def step(i):
        h.copy_(h0[i % POOL].view(1, -1))
        moe.stack_forward(shape, h, wrs, bs, Ws, ws)

    if persistent:
        return _run_stack_persistent(hip, steps, warmup, s, shape, h, h0, wrs, bs, Ws, keep, stream)

    # timed as replays of one captured graph of the 43 layers; the fresh token is copied in
    # before each replay (inside the timed region)
    step(0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        moe.stack_forward(shape, h, wrs, bs, Ws, ws)
    torch.cuda.synchronize()

    def step_graph(i):
        h.copy_(h0[i % POOL].view(1, -1))
        graph.replay()

    total, groups = _timed(hip, stream, step_graph, steps, warmup)
    # the timing hook's events ride on eager launches
    _, k_up = _timed(hip, stream, step, steps, warmup, profile=moe.KERNEL_FFN_UP)
    _, k_down = _timed(hip, stream, step, steps, warmup, profile=moe.KERNEL_FFN_DOWN)
    ms = total / steps
    up_b, down_b = expert_bytes(s)
    # T = 1, k = 6 distinct experts per layer
    layer_bytes = s.k * (up_b + down_b)
    rec = dict(workload="c4_stack", desc=WORKLOADS["c4_stack"][3], T=1, ms_per_step=ms, tokens_per_s=1.0 / (ms * 1e-3),
               ms_per_step_median_of_5=float(np.median(groups)),
               bound="hbm", alg_bytes_per_step=float(layer_bytes * s.n_layers),
               step_GBps=layer_bytes * s.n_layers / (ms * 1e-3) / 1e9,
               ffn_up_us=float(np.mean(k_up) * 1e3), ffn_down_us=float(np.mean(k_down) * 1e3) if k_down else None)
    rec["step_frac_hbm"] = rec["step_GBps"] / HBM_PEAK_GBS
    # the hook's events bracket the last layer's launch of the step only
    rec["ffn_up_alg_bytes"] = float(s.k * up_b)
    rec["ffn_up_GBps"] = s.k * up_b / (np.mean(k_up) * 1e-3) / 1e9
    rec["ffn_up_frac"] = rec["ffn_up_GBps"] / HBM_PEAK_GBS
    del keep, Ws, wrs, bs, ws
    moe._ws_cache.clear()
    torch.cuda.empty_cache()
    return rec


def _run_stack_persistent(hip, steps, warmup, s, shape, h, h0, wrs, bs, Ws, keep, stream):
    """The same stack as one cooperative launch per token (moe_stack_forward_persistent), launched
    eagerly; the fresh token is copied in before each launch (inside the timed region)."""
    import torch
    import sparse_mixture_experts_16_amd as moe
    pws = torch.empty(moe.stack_persistent_workspace_size(shape, s.n_layers), dtype=torch.uint8, device="cuda")

    def step(i):
        h.copy_(h0[i % POOL].view(1, -1))
        moe.stack_forward_persistent(shape, h, wrs, bs, Ws, pws)

    total, groups = _timed(hip, stream, step, steps, warmup)
    if moe.stack_persistent_status(pws) != 0:
        raise RuntimeError("persistent stack: a grid-barrier wait ran out")
    ms = total / steps
    up_b, down_b = expert_bytes(s)
    layer_bytes = s.k * (up_b + down_b)
    step_bytes = float(layer_bytes * s.n_layers)
    rec = dict(workload="c4_stack_persistent", desc=WORKLOADS["c4_stack_persistent"][3], T=1, ms_per_step=ms,
               ms_per_step_median_of_5=float(np.median(groups)),
               tokens_per_s=1.0 / (ms * 1e-3), bound="hbm", alg_bytes_per_step=step_bytes,
               step_GBps=step_bytes / (ms * 1e-3) / 1e9)
    rec["step_frac_hbm"] = rec["step_GBps"] / HBM_PEAK_GBS
    # one kernel does the whole step: its roofline is the step's (the launch also holds the
    # barrier-word clear and the token copy)
    rec.update(ffn_up_alg_bytes=step_bytes, ffn_up_us=ms * 1e3, ffn_up_GBps=rec["step_GBps"],
               ffn_up_frac=rec["step_frac_hbm"], roof_kernel="dec_stack (the whole 43-layer step, one launch)")
    del keep, Ws, wrs, bs, pws
    moe._ws_cache.clear()
    torch.cuda.empty_cache()
    return rec


def _to_dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


# ------------------------------------------------------------------------------------------------
# Device peaks (libmoe_peaks.so)
# ------------------------------------------------------------------------------------------------
def measure_peaks(hip):
    """The HBM read stream over a 4 GiB buffer (far beyond the 256 MB Infinity Cache), the same
    stream cut into 80 MB reads (one decode layer's weights), and the bf16 and fp8 x fp4 matrix
    instructions on register operands, each the best of a few launch shapes."""
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_mixture_experts_16_amd", "libmoe_peaks.so"))
    lib.peak_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    stream = torch.cuda.current_stream().cuda_stream
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(7)
    out = torch.empty(cus * 64 * 256, dtype=torch.float32, device="cuda")

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = hip.event(), hip.event()
        hip.record(e0, stream)
        for r in range(reps):
            fn(r)
        hip.record(e1, stream)
        ms = hip.elapsed_ms(e0, e1) / reps
        hip.destroy(e0)
        hip.destroy(e1)
        return ms

    res = {}
    best = 0.0
    for bpc in (4, 8, 16):
        ms = timed(lambda r=0: lib.peak_hbm_read(buf.data_ptr(), nbytes, cus * bpc, out.data_ptr(), stream), 5)
        best = max(best, nbytes / (ms * 1e-3) / 1e9)
    res["hbm_read_GBps"] = best
    win = 80 << 20  # one MXFP4 decode layer's active-expert bytes, read from a moving place
    nwin = nbytes // win
    best = 0.0
    for bpc in (2, 4, 8):
        ms = timed(lambda r=0: lib.peak_hbm_read(buf.data_ptr() + (r % nwin) * win, win, cus * bpc, out.data_ptr(),
                                                 stream), 2 * nwin)
        best = max(best, win / (ms * 1e-3) / 1e9)
    res["hbm_read_80MB_GBps"] = best
    nacc = 8
    for kind, name, kdim in ((0, "bf16_TFLOPs", 16), (1, "fp8xfp4_TFLOPs", 64)):
        best = 0.0
        for wgs in (1, 2):
            iters = 2000
            ms = timed(lambda r=0: lib.peak_mfma(kind, cus * wgs, iters, out.data_ptr(), stream), 3)
            flops = cus * wgs * 4 * iters * nacc * 2.0 * 32 * 32 * kdim
            best = max(best, flops / (ms * 1e-3) / 1e12)
        res[name] = best
    del buf, out
    torch.cuda.empty_cache()
    return res


def roofline(rec, peaks):
    """The roofline object of one workload: its dominant kernel (the gate/up FFN kernel) against
    the spec peak and the measured one, with the whole step's fraction beside it."""
    mx = rec["workload"] in MX_WORKLOADS
    if rec["bound"] == "hbm":
        r = dict(bound="hbm", achieved=rec["ffn_up_GBps"], peak=HBM_PEAK_GBS, unit="GB/s", frac=rec["ffn_up_frac"],
                 traffic=traffic_bytes(rec["workload"]),
                 kernel=rec.get("roof_kernel", "FFN gate/up + SwiGLU (decode grouped GEMV)"),
                 alg_bytes_per_launch=rec["ffn_up_alg_bytes"], avg_launch_us=rec["ffn_up_us"],
                 step_frac=rec["step_frac_hbm"])
        if peaks:
            r["measured_peak"] = peaks["hbm_read_GBps"]
            r["frac_of_measured_peak"] = rec["ffn_up_GBps"] / peaks["hbm_read_GBps"]
            r["step_frac_of_measured_peak"] = rec["step_GBps"] / peaks["hbm_read_GBps"]
    else:
        peak = FP8_PEAK_TFLOPS if mx else BF16_PEAK_TFLOPS
        r = dict(bound="mfma", achieved=rec["ffn_up_TFLOPs"], peak=peak, unit="TFLOP/s", frac=rec["ffn_up_frac"],
                 traffic=traffic_bytes(rec["workload"]),
                 kernel="FFN gate/up + SwiGLU (prefill grouped MFMA GEMM" + (", fp8 x fp4)" if mx else ", bf16)"),
                 alg_flops_per_launch=rec["ffn_up_alg_flops"], avg_launch_us=rec["ffn_up_us"],
                 step_frac=rec["step_frac_mfma"])
        if peaks:
            mp = peaks["fp8xfp4_TFLOPs" if mx else "bf16_TFLOPs"]
            r["measured_peak"] = mp
            r["frac_of_measured_peak"] = rec["ffn_up_TFLOPs"] / mp
            r["step_frac_of_measured_peak"] = rec["step_TFLOPs"] / mp
    return r


# ------------------------------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on bounded samples of each workload
# ------------------------------------------------------------------------------------------------
_host_expert_cache = {}


def _host_experts_cached(s, layer, experts):
    """Host weights of the listed experts (generated once per (config, layer, expert))."""
    import moe_inputs as mi
    missing = [e for e in experts if (s.name, layer, e) not in _host_expert_cache]
    if missing:
        w = mi.host_experts(s, layer, experts=missing)
        for i, e in enumerate(missing):
            _host_expert_cache[(s.name, layer, e)] = {k: (v[i] if isinstance(v, np.ndarray) else v) for k, v in w.items()}
    parts = [_host_expert_cache[(s.name, layer, e)] for e in experts]
    return {k: (np.ascontiguousarray(np.stack([p[k] for p in parts])) if isinstance(parts[0][k], np.ndarray)
                else parts[0][k]) for k in parts[0]}


def _oracle_layer_run(s, x, wr, b, layer=0, flags=0, h=None):
    """Prepare one oracle evaluation of the layer on the token rows x (or, with h, of the stack
    layer on the residual rows h): the router over all E experts, the FFNs of the selected experts
    (generated here, outside the timed call).  Returns the timed callable."""
    import moe_inputs as mi
    import oracle
    xin = oracle.rmsnorm(h, dtype=s.act) if h is not None else x
    l32, _ = oracle.router_logits(s, xin, wr, b)
    idx, _ = oracle.topk(s, l32)
    need = sorted(set(idx.reshape(-1).tolist()))
    w = _host_experts_cached(s, layer, need)
    sh = mi.host_experts(s, layer, shared=True) if s.n_shared else None
    remap = np.full(s.E, -1, np.int64)
    remap[need] = np.arange(len(need))

    def run():
        xr = oracle.rmsnorm(h, dtype=s.act) if h is not None else x
        l32r, _ = oracle.router_logits(s, xr, wr, b)
        ir, g = oracle.topk(s, l32r)
        ic = remap[ir].astype(np.int32)
        sc = mi.LayerSpec(s.name, xr.shape[0], s.d, s.f, len(need), s.k, s.n_shared, s.f_shared, s.act, s.wt,
                          s.sigma_x, s.sigma_w, s.sigma_r)
        _, o, p, iv = oracle.permute(sc, ic)
        ys, ysh = oracle.grouped_ffn(sc, xr, p, o, w, sh, flags=flags)
        return oracle.combine(sc, ys, iv, ic, g, ysh)
    return run


def cpu_baseline(name: str, seconds: float):
    """tokens/s of the oracle on a bounded sample of workload `name`: the sample's token batches
    are drawn like the benchmark's (decode: the pool's batches in turn; prefill: single tokens of
    the batch, whose rows are independent); each batch's selected experts are generated before its
    timed call."""
    import moe_inputs as mi
    import oracle
    cfg, T, _, desc = WORKLOADS[name] if name in WORKLOADS else CPU_ONLY[name]
    mx = name in MX_WORKLOADS
    flags = oracle.MX_GEMM if mx else 0
    if cfg == "c4":
        s = mi.spec("c4")
        h0 = mi.host_h0(mi.spec("c4", T=1))
        per_layer = []
        for layer in (0, 21, 42):
            wr, b = mi.host_router(s, layer)
            run = _oracle_layer_run(s, None, wr, b, layer=layer, h=h0)
            t0 = time.perf_counter()
            n = 0
            while n < 1 or time.perf_counter() - t0 < seconds / 3:
                run()
                n += 1
            per_layer.append((time.perf_counter() - t0) / n)
        step = float(np.mean(per_layer)) * s.n_layers
        return dict(value=1.0 / step, unit="tokens/s", cores=oracle.num_threads(), kind="oracle",
                    sample=f"one token through layers 0, 21 and 42 of the stack ({', '.join(f'{t * 1e3:.0f}' for t in per_layer)} "
                           f"ms each, the six selected experts of each generated beforehand), mean x 43 layers: extrapolated")
    s = mi.spec(cfg, T=T)
    wr, b = mi.host_router(s)
    decode = T <= 32
    rows = T if decode else 1
    xs = mi.host_x(mi.spec(cfg, T=max(64, rows * 4)))
    done = tokens = 0
    busy = 0.0
    t_wall = time.perf_counter()
    while (done < 1 or busy < seconds) and time.perf_counter() - t_wall < 4 * seconds:
        x = np.ascontiguousarray(xs[(done * rows) % len(xs):(done * rows) % len(xs) + rows])
        run = _oracle_layer_run(s, x, wr, b, flags=flags)
        t0 = time.perf_counter()
        run()
        busy += time.perf_counter() - t0
        done += 1
        tokens += rows
    what = f"{done} batches of {rows} token(s)" if decode else f"{done} single tokens of the T={T} batch"
    return dict(value=tokens / busy, unit="tokens/s", cores=oracle.num_threads(), kind="oracle",
                sample=f"{what}: {desc}; {busy:.1f} s of timed fp64 CPU work (expert weights generated beforehand)")


def cpu_single_thread(names, seconds):
    """The oracle's single-threaded rates, each in a child process with OMP_NUM_THREADS=1."""
    import subprocess
    out = {}
    for n in names:
        env = dict(os.environ, OMP_NUM_THREADS="1")
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-only", n, "--cpu-seconds", str(seconds)],
                           capture_output=True, text=True, env=env, timeout=600)
        try:
            out[n] = json.loads(r.stdout.strip().splitlines()[-1])
        except Exception:  # keep the line printable
            out[n] = {"error": (r.stderr or r.stdout)[-300:]}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(WORKLOADS))
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-peaks", action="store_true")
    ap.add_argument("--sweep-list", default="")
    ap.add_argument("--cpu-only", default="", help="print only the oracle's rate on this workload (no GPU)")
    ap.add_argument("--cpu-seconds", type=float, default=3.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a 256 MiB device copy (reference for the traffic counters)")
    args = ap.parse_args()
    if args.cpu_only:
        print(json.dumps(cpu_baseline(args.cpu_only, args.cpu_seconds)))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1 "
                                   "(the layer's multi-GPU sharding is a design note, not built)"}))
        sys.exit(2)
    import torch
    if args.copy_calibration:
        copy_calibration()
        return
    import sparse_mixture_experts_16_amd  # noqa: F401  (fails loudly without the HIP library)
    hip = Hip()
    torch.cuda.init()
    peaks = None
    if not args.no_peaks:
        print("[bench] device peaks ...", file=sys.stderr, flush=True)
        peaks = measure_peaks(hip)

    def run(name, steps, warmup):
        print(f"[bench] {name} ...", file=sys.stderr, flush=True)
        if name in ("c4_stack", "c4_stack_persistent"):
            rec = run_stack_workload(hip, steps, warmup, persistent=name == "c4_stack_persistent")
        else:
            rec = run_layer_workload(hip, name, steps, warmup)
        rec["roofline"] = roofline(rec, peaks)
        return rec

    head = run(args.workload, args.steps, args.warmup)
    sweep = {}
    if not args.no_sweep:
        names = [n for n in (args.sweep_list.split(",") if args.sweep_list else WORKLOADS) if n and n != args.workload]
        for n in names:
            try:
                sweep[n] = run(n, args.steps, args.warmup)
            except Exception as exc:  # keep the line printable; the failure is reported in it
                sweep[n] = {"error": repr(exc)}
                print(f"[bench] {n} failed: {exc!r}", file=sys.stderr, flush=True)
    cpu = cpu_single = None
    if not args.no_cpu:
        print("[bench] oracle on the host ...", file=sys.stderr, flush=True)
        cpu = cpu_baseline(head["workload"], 12.0)
        for n, rec in sweep.items():
            if "error" not in rec:
                rec["cpu_baseline"] = cpu_baseline(n, 2.0)
        cpu_single = cpu_single_thread(["c0_tiny_T16", "c1_decode_T1", "c3_decode_T1"], 3.0)
    line = {
        "metric": "MoE-layer tokens/s; decode HBM GB/s % peak; prefill MFMA util %",
        "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "ms_per_step_median_of_5": head.get("ms_per_step_median_of_5"), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": head["desc"], "name": head["workload"], "T": head["T"],
                   **{key: head[key] for key in ("experts_hit_per_step", "step_GBps", "step_frac_hbm",
                                                 "step_TFLOPs", "step_frac_mfma") if key in head}},
        "roofline": head["roofline"], "cpu_baseline": cpu,
        "cpu_single_thread": cpu_single,
        "measured_peaks": peaks,
        "kernels_us": {key: head[key] for key in ("ffn_up_us", "ffn_down_us") if key in head},
        "sweep": sweep,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
