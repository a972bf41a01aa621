"""Build libmoe.so (the C-ABI library of hand-written gfx950 HIP kernels).

    python -m latent_mixture_experts_amd.build

Compiles every ``csrc/*.hip`` for gfx950 with hipcc (one object per source,
in parallel) and links them into ``latent_mixture_experts_amd/libmoe.so``. Packed-fp32 instruction selection is
turned off for all device code (``-packed-fp32-ops``).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmoe.so")
PEAKS_SRC = os.path.join(HERE, "peaks", "peaks.hip")
PEAKS_LIB = os.path.join(HERE, "libmoe_peaks.so")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _filter(stderr: str) -> str:
    # hipcc's host pass does not know the device-only feature flag: drop that note
    noise = "is not a recognized feature for this target"
    return "\n".join(l for l in stderr.splitlines() if noise not in l)


def build(verbose: bool = False) -> str:
    """Always compiles (the build check): every source to an object in
    parallel, then one link; atomically replaces libmoe.so."""
    import concurrent.futures
    import tempfile

    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    compile_flags = [f for f in FLAGS if f != "-shared"]
    with tempfile.TemporaryDirectory(prefix="moe_build_") as tmpdir:
        objs = []
        cmds = []
        for src in sources():
            obj = os.path.join(tmpdir, os.path.basename(src)[:-4] + ".o")
            objs.append(obj)
            cmds.append([hipcc, *compile_flags, "-c", src, "-o", obj])
        jobs = max(1, min(len(cmds), os.cpu_count() or 1, 16))
        with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(lambda c: subprocess.run(c, capture_output=True, text=True), cmds))
        for c, r in zip(cmds, results):
            err = _filter(r.stderr)
            if verbose:
                print(" ".join(c), flush=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed ({r.returncode}) on {c[-3]}:\n{err}")
            if err.strip() and verbose:
                print(err, file=sys.stderr)
        tmp = LIB + ".tmp"
        link = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
        r = subprocess.run(link, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc link failed ({r.returncode}):\n{_filter(r.stderr)}")
    os.replace(tmp, LIB)
    return LIB


def build_peaks() -> str:
    """libmoe_peaks.so: the benchmark's measurement kernels (copy, read and
    MFMA ceilings), a library of its own."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = PEAKS_LIB + ".tmp"
    r = subprocess.run([hipcc, *FLAGS, PEAKS_SRC, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}) on {PEAKS_SRC}:\n{_filter(r.stderr)}")
    os.replace(tmp, PEAKS_LIB)
    return PEAKS_LIB


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_peaks())
