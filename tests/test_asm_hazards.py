"""Wait states before the GEMM kernels' inline-assembly LDS DMA instructions (host-only check of
the gfx950 assembly the compiler emits for csrc/gemm.hip).

The global -> LDS DMA is written as inline assembly, so the compiler schedules around it without
knowing what it is and inserts none of the wait states the hardware requires before it. Two
hazards apply: a VALU instruction (e.g. v_readfirstlane) that writes an SGPR the DMA reads as its
base address needs 5 wait states before the DMA, and a write of M0 (the DMA's LDS address) needs
1. Too few of the former let the DMA use a stale base address (a GPU memory fault). This test
compiles the kernels to assembly and checks every DMA site.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "fp8_blockwise_quantization_amd", "csrc", "gemm.hip")

VALU_SGPR_WAIT = 5
M0_WAIT = 1


def _hipcc():
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return None


def _sgprs(op):
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", op)
    if m:
        return {f"s{k}" for k in range(int(m.group(1)), int(m.group(2)) + 1)}
    return {op}


def _instructions(text):
    out = []
    for line in text.split("\n"):
        t = line.split(";")[0].strip()
        if not t or t.startswith(".") or t.endswith(":"):
            continue
        out.append(t)
    return out


def _waits(ins):
    m = re.match(r"s_nop\s+(\d+)", ins)
    return int(m.group(1)) + 1 if m else 1


def dma_hazards(asm_text):
    """(site, reason) for every LDS DMA with too few wait states after a write of its operands."""
    ins = _instructions(asm_text)
    bad = []
    for i, t in enumerate(ins):
        m = re.match(r"global_load_lds_dword\w*\s+v\d+,\s*(s\[\d+:\d+\])", t)
        if not m:
            continue
        base = _sgprs(m.group(1))
        waited, j = 0, i - 1
        while j >= 0 and waited < VALU_SGPR_WAIT:
            prev = ins[j]
            d = re.match(r"(\w+)\s+([^,\s]+)", prev)
            if d:
                op, dst = d.group(1), d.group(2)
                if op.startswith("v_") and _sgprs(dst) & base:
                    bad.append((t, f"VALU write of {dst} {waited} wait states before"))
                if dst == "m0" and waited < M0_WAIT:
                    bad.append((t, f"M0 written {waited} wait states before"))
            waited += _waits(prev)
            j -= 1
    return bad


def test_detector_flags_a_readfirstlane_right_before_the_dma():
    asm = "\n".join(["v_readfirstlane_b32 s20, v2", "v_readfirstlane_b32 s21, v3",
                     "global_load_lds_dword v1, s[20:21]"])
    assert len(dma_hazards(asm)) == 2
    ok = "\n".join(["v_readfirstlane_b32 s20, v2", "s_mov_b32 m0, s4", "s_nop 4",
                    "global_load_lds_dwordx4 v1, s[20:21]"])
    assert dma_hazards(ok) == []


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_every_gemm_dma_site_has_its_wait_states(tmp_path):
    out = tmp_path / "gemm.s"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
           "--cuda-device-only", "-S", "-o", str(out), SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    text = out.read_text()
    sites = len(re.findall(r"global_load_lds_dword", text))
    assert sites > 100  # the DMA-fed kernels are in the file
    bad = dma_hazards(text)
    assert bad == [], f"{len(bad)} DMA sites lack wait states, e.g. {bad[:3]}"
