"""Register budgets of the hot kernels, read from the compiler's resource
report for gfx950 (hipcc -Rpass-analysis=kernel-resource-usage): the
prefill expert kernels (MXFP4 and NVFP4) must keep two workgroups of eight
wavefronts per CU (at most 128 VGPRs: at 130 the MXFP4 one ran gate/up 45%
slower at T = 4096; the NVFP4 one at 145 VGPRs ran at 0.62x MXFP4's rate,
at 119 at 0.86x), and no hot kernel may spill to scratch in its loop. CPU
only (compiles, runs nothing)."""
from __future__ import annotations

import re
import shutil
import subprocess

import pytest

from latent_mixture_experts_amd import build as B

HIPCC = "/opt/rocm/bin/hipcc"
pytestmark = pytest.mark.skipif(shutil.which(HIPCC) is None, reason="hipcc not installed")


def _report(src: str) -> dict[str, dict[str, int]]:
    flags = [f for f in B.FLAGS if f != "-shared"]
    r = subprocess.run([HIPCC, *flags, "-Rpass-analysis=kernel-resource-usage", "--offload-device-only",
                        "-c", f"{B.CSRC}/{src}", "-o", "/dev/null"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            out[cur] = {}
            continue
        for key, pat in (("vgpr", r"VGPRs: (\d+)"), ("scratch", r"ScratchSize \[bytes/lane\]: (\d+)"),
                         ("waves", r"Occupancy \[waves/SIMD\]: (\d+)")):
            m = re.search(pat, line)
            if m and cur:
                out[cur][key] = int(m.group(1))
    return out


def test_prefill_expert_kernel_keeps_two_workgroups_per_cu():
    rep = _report("gemm_expert.hip")
    fp4 = {k: v for k, v in rep.items() if "expert_kernelILi1E" in k or "expert_kernelILi2E" in k}
    assert len(fp4) == 4, list(rep)  # MXFP4 and NVFP4, gate/up and down
    for name, v in fp4.items():
        assert v["vgpr"] <= 128 and v["waves"] >= 4 and v["scratch"] == 0, (name, v)
    for name, v in rep.items():
        assert v["scratch"] == 0, (name, v)


def test_decode_streaming_kernels_keep_their_occupancy():
    """Every FP4 streaming kernel with its rows staged in LDS (the form the
    layer runs at these widths; rows in registers only when they exceed the
    LDS) keeps two workgroups per CU and does not spill, but for the NVFP4
    few-rows form with a K split and two weight stages in flight, whose 12
    bytes per lane go to scratch outside its main loop. (A spill of a
    loaded value makes a pass wait for it before it issues its weight
    loads: the NVFP4 kernels spilled their early activation pieces until the
    wavefront index was made scalar and the rows were copied straight into
    LDS.)"""
    rep = _report("gemm_skinny.hip")
    fp4 = {k: v for k, v in rep.items()
           if re.search(r"stream_kernelILi[1-4]E", k) and k.endswith("Lb1EEEvNS_10SkinnyArgsE")}
    assert len(fp4) >= 40, list(rep)[:5]
    for name, v in fp4.items():
        assert v["waves"] >= 4, (name, v)
        assert v["scratch"] <= (16 if "stream_kernelILi3E" in name else 0), (name, v)
