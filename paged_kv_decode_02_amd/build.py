"""Build libpakv.so in-tree with hipcc for gfx950.

    python -m paged_kv_decode_02_amd.build

Extra ``-D`` defines (split geometry) can be passed to ``build(defines=...)``.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libpakv.so"
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpakv)")


def build(out_path: str | None = None, defines=(), verbose: bool = False) -> str:
    """Compile csrc/pakv.hip (kernels and their host side) and csrc/pakv_sched.cpp
    (host page allocator) into one shared library; returns its path."""
    out_path = out_path or os.path.join(HERE, LIB_NAME)
    tmp = out_path + ".tmp"
    cmd = [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
        # packed FP32 instructions are kept out of the device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # keep MFMA accumulators in ordinary VGPRs (the softmax rescales them)
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-Wno-unused-command-line-argument",
        f"-I{INCLUDE}", f"-I{CSRC}",
        *[f"-D{d}" for d in defines],
        os.path.join(CSRC, "pakv.hip"),
        os.path.join(CSRC, "pakv_sched.cpp"),
        "-Wl,-rpath,/opt/rocm/lib",
        "-o", tmp,
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")
    os.replace(tmp, out_path)
    return out_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
