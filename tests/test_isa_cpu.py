"""Code-generation guard for the grouped-GEMM pipelines (CPU only: hipcc cross-compiles gfx950).

Both GEMMs fill an LDS ring with global_load_lds and order each stage's loads before its fragment
reads with explicit vmcnt waits and barriers.  The compiler inserts waits of its own before an LDS
read that may alias an LDS-DMA store; if it cannot rule that out (e.g. a read through a struct type
carrying no type-based alias information), it waits for every load in flight, which silently
serialises the ring (the MX kernel ran that way, 20% slower).  This test compiles both sources to
gfx950 assembly and checks that no vmcnt wait sits directly before an LDS read in any grouped-GEMM
kernel.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "sparse_mixture_experts_16_amd", "csrc")
INC = os.path.join(HERE, "..", "include")

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None, reason="needs hipcc")


def _kernels(src: str, prefix: str, tmp_path) -> dict[str, list[str]]:
    from sparse_mixture_experts_16_amd import _build
    out = tmp_path / (src + ".s")
    flags = [f for f in _build.HIPCC_FLAGS if f != "-fPIC"]
    r = subprocess.run(["hipcc", *flags, "--offload-device-only", "-S", "-I", CSRC, "-I", INC, "-o", str(out),
                        os.path.join(CSRC, src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    text = out.read_text()
    kernels = {}
    for m in re.finditer(rf"^({prefix}\S*):", text, re.M):
        body = text[m.end():text.index("s_endpgm", m.end())]
        kernels[m.group(1)] = [ln.strip() for ln in body.split("\n") if ln.strip() and not ln.strip().startswith(";")]
    return kernels


def _drains(lines: list[str]) -> list[str]:
    """vmcnt waits whose next instruction reads LDS, in stretches that follow a global_load_lds."""
    bad, after_dma = [], False
    for a, b in zip(lines, lines[1:]):
        if a.startswith("global_load_lds"):
            after_dma = True
        if after_dma and a.startswith("s_waitcnt") and "vmcnt" in a and b.startswith("ds_read"):
            bad.append(f"{a} -> {b}")
    return bad


@pytest.mark.parametrize("src,prefix", [("mxgemm.hip", "_ZN3moe6mxgemm"), ("gemm.hip", "_ZN3moe5ggemm"),
                                        ("gemm.hip", "_ZN3moe9ggemm_w2q")])
def test_no_compiler_drain_before_fragment_reads(src, prefix, tmp_path):
    kernels = _kernels(src, prefix, tmp_path)
    assert kernels, f"no {prefix} kernels found in {src}"
    for name, lines in kernels.items():
        assert any(ln.startswith("global_load_lds") for ln in lines), name
        assert not _drains(lines), (name, _drains(lines)[:4])


def test_persistent_stack_keeps_its_prefetch_in_flight(tmp_path):
    """The persistent decode stack issues the down projection's weight rows right after the routing,
    to land under the gate/up stream.  A flat load (a read of the LDS routing table through a
    pointer the compiler cannot place in LDS) or a scratch reload (a register spill) makes the
    compiler wait for every global load in flight before using it, which serialised that prefetch
    row by row (routing phase 4.3 -> 10.3 us).  Neither may appear in the kernel."""
    kernels = _kernels("decode.hip", "_ZN3moe9dec_stack", tmp_path)
    assert kernels, "no dec_stack kernel found in decode.hip"
    for name, lines in kernels.items():
        flat = [ln for ln in lines if ln.startswith("flat_load")]
        scratch = [ln for ln in lines if ln.startswith("scratch_") or ln.startswith("buffer_") and "off, s[0:3]" in ln]
        assert not flat, (name, flat[:4])
        assert not scratch, (name, scratch[:4])
        assert any(ln.startswith("global_load_dwordx4") for ln in lines), name
