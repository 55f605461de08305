"""Benchmark of the routed MoE layer on one MI355X through the C-ABI library.

A step is one pass of the whole layer (router logits, top-k + gates, permute, grouped
expert FFNs, combine; for the stack, 43 such layers with the RMS-norm residual glue)
over one batch of synthetic tokens already resident in HBM.  The headline workload is
the decode layer of the 128-expert top-8 + shared bf16 configuration at T=1; the other
workloads run as a sweep and are reported beside it in the same JSON line.

Decode steps draw a fresh token batch from a pool of 256 batches and rotate through
several copies of the layer's weights (like successive layers of a model), so the
256 MB Infinity Cache cannot serve repeated weight reads.

Timing: hipEvents on the stream the library launches on (torch's current stream).
Pass 1 times K steps end to end (value, ms_per_step).  Pass 2 repeats K steps with the
library's timing hook bracketing the gate/up FFN kernel (the largest share of the
layer's bytes and flops) to get that kernel's average duration for the roofline.

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
}
HEADLINE = "c1_decode_T1"
MX_WORKLOADS = {"c3_prefill_mx"}  # run with MOE_F_MX_GEMM
POOL = 256

# HBM traffic of the roofline kernel, from two rocprofv3 --pmc passes (FETCH_SIZE, then
# WRITE_SIZE, KiB per dispatch, averaged over the dispatches of the bench command) scaled by
# what the same counters read for a plain device-to-device copy of 256 MiB.  Each entry names
# the digest of the kernel sources it was taken on; a different digest reports null.
KERNEL_SOURCES = {
    "decode": ["decode.hip", "common.h", "wchunk.h"],
    "gemm": ["gemm.hip", "common.h", "wchunk.h", "lds_dma.h"],
    "mx": ["mxgemm.hip", "common.h", "lds_dma.h"],
}
COPY_CAL = dict(fetch_factor=1.99981, write_factor=1.00000)
TRAFFIC = {  # workload -> counters of its roofline kernel (profiles/<kernel>__<workload>.txt)
    "c1_decode_T1": dict(src="decode:c5b63d35f7ebcacf", fetch_kib=27752.8, write_kib=54.3),
    "c3_decode_T1": dict(src="decode:c5b63d35f7ebcacf", fetch_kib=26256.3, write_kib=96.8),
    "c3nv_decode_T1": dict(src="decode:c5b63d35f7ebcacf", fetch_kib=27789.2, write_kib=96.2),
    "c4_stack": dict(src="decode:c5b63d35f7ebcacf", fetch_kib=26256.1, write_kib=96.7),
    "c2_prefill": dict(src="gemm:3a79fcd2ca97bd29", fetch_kib=762210.1, write_kib=110592.0),
    "c3_prefill": dict(src="gemm:3a79fcd2ca97bd29", fetch_kib=1327013.7, write_kib=393216.0),
    "c3_prefill_mx": dict(src="mx:81115b7c99f1254b", fetch_kib=1377996.2, write_kib=102178.8),
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
    """A plain 256 MiB device-to-device copy, 5 times (the counters' reference)."""
    import torch
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 5}))


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


def _timed(hip, stream, step, steps, warmup, profile=None):
    """Run warmup + timed steps; returns total ms (and per-step kernel ms if profiling)."""
    import torch
    import sparse_mixture_experts_16_amd as moe
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    kern = []
    if profile is None:
        e0, e1 = hip.event(), hip.event()
        hip.record(e0, stream)
        for i in range(steps):
            step(warmup + i)
        hip.record(e1, stream)
        torch.cuda.synchronize()
        total = hip.elapsed_ms(e0, e1)
        hip.destroy(e0)
        hip.destroy(e1)
        return total, kern
    evs = [(hip.event(), hip.event()) for _ in range(steps)]
    for i in range(steps):
        moe.profile_kernel(profile, evs[i][0], evs[i][1])
        step(warmup + i)
    moe.profile_kernel(-1)
    torch.cuda.synchronize()
    for a, b in evs:
        kern.append(hip.elapsed_ms(a, b))
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

    total, _ = _timed(hip, stream, step, steps, warmup)
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
               ffn_up_us=float(np.mean(k_up) * 1e3), ffn_down_us=float(np.mean(k_down) * 1e3),
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


def run_stack_workload(hip, steps, warmup):
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

    total, _ = _timed(hip, stream, step_graph, steps, warmup)
    # the timing hook's events ride on eager launches
    _, k_up = _timed(hip, stream, step, steps, warmup, profile=moe.KERNEL_FFN_UP)
    _, k_down = _timed(hip, stream, step, steps, warmup, profile=moe.KERNEL_FFN_DOWN)
    ms = total / steps
    up_b, down_b = expert_bytes(s)
    # T = 1, k = 6 distinct experts per layer
    layer_bytes = s.k * (up_b + down_b)
    rec = dict(workload="c4_stack", desc=WORKLOADS["c4_stack"][3], T=1, ms_per_step=ms, tokens_per_s=1.0 / (ms * 1e-3),
               bound="hbm", alg_bytes_per_step=float(layer_bytes * s.n_layers),
               step_GBps=layer_bytes * s.n_layers / (ms * 1e-3) / 1e9,
               ffn_up_us=float(np.mean(k_up) * 1e3), ffn_down_us=float(np.mean(k_down) * 1e3))
    rec["step_frac_hbm"] = rec["step_GBps"] / HBM_PEAK_GBS
    # the hook's events bracket the last layer's launch of the step only
    rec["ffn_up_alg_bytes"] = float(s.k * up_b)
    rec["ffn_up_GBps"] = s.k * up_b / (np.mean(k_up) * 1e-3) / 1e9
    rec["ffn_up_frac"] = rec["ffn_up_GBps"] / HBM_PEAK_GBS
    del keep, Ws, wrs, bs, ws
    moe._ws_cache.clear()
    torch.cuda.empty_cache()
    return rec


def _to_dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def cpu_baseline(seconds: float = 12.0):
    """The oracle, as it stands, on the headline workload: C1 decode layer, one token at a time."""
    import moe_inputs as mi
    import oracle
    s = mi.spec("c1", T=1)
    wr, b = mi.host_router(s)
    w = mi.host_experts(s)
    sh = mi.host_experts(s, shared=True)
    xs = mi.host_x(mi.spec("c1", T=POOL))
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        oracle.layer_forward(s, np.ascontiguousarray(xs[n % POOL:n % POOL + 1]), wr, b, w, sh)
        n += 1
    dt = time.perf_counter() - t0
    return dict(value=n / dt, unit="tokens/s", cores=oracle.num_threads(), kind="oracle",
                sample=f"{n} single-token decode layers of the bf16 E=128 top-8 + shared layer (d=2048, f=768), "
                       f"{dt:.1f} s of fp64 CPU work")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(WORKLOADS))
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--sweep-list", default="")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a 256 MiB device copy (reference for the traffic counters)")
    args = ap.parse_args()
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

    def run(name, steps, warmup):
        print(f"[bench] {name} ...", file=sys.stderr, flush=True)
        if name == "c4_stack":
            return run_stack_workload(hip, steps, warmup)
        return run_layer_workload(hip, name, steps, warmup)

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
    cpu = None if args.no_cpu else cpu_baseline()
    if head["bound"] == "hbm":
        roof = dict(bound="hbm", achieved=head["ffn_up_GBps"], peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=head["ffn_up_frac"], traffic=traffic_bytes(head["workload"]), kernel="FFN gate/up + SwiGLU (decode grouped GEMV)",
                    alg_bytes_per_launch=head["ffn_up_alg_bytes"], avg_launch_us=head["ffn_up_us"])
    else:
        roof = dict(bound="mfma", achieved=head["ffn_up_TFLOPs"],
                    peak=FP8_PEAK_TFLOPS if head["workload"] in MX_WORKLOADS else BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=head["ffn_up_frac"], traffic=traffic_bytes(head["workload"]), kernel="FFN gate/up + SwiGLU (prefill grouped MFMA GEMM)",
                    alg_flops_per_launch=head["ffn_up_alg_flops"], avg_launch_us=head["ffn_up_us"])
    line = {
        "metric": "MoE-layer tokens/s; decode HBM GB/s % peak; prefill MFMA util %",
        "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": head["desc"], "name": head["workload"], "T": head["T"],
                   **{key: head[key] for key in ("experts_hit_per_step", "step_GBps", "step_frac_hbm",
                                                 "step_TFLOPs", "step_frac_mfma") if key in head}},
        "roofline": roof, "cpu_baseline": cpu,
        "kernels_us": {key: head[key] for key in ("ffn_up_us", "ffn_down_us") if key in head},
        "sweep": sweep,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
