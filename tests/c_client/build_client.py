"""Build step for the plain C clients of libpakv (test infrastructure):
gcc, C11, the HIP runtime's C API and libpakv.so from the package directory:
the program pakv_client and the HIP-graph step driver libpakv_graph.so.

    python tests/c_client/build_client.py
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "paged_kv_decode_02_amd")
SRC = os.path.join(HERE, "pakv_client.c")
OUT = os.path.join(HERE, "pakv_client")


GRAPH_SRC = os.path.join(HERE, "pakv_graph.c")
GRAPH_OUT = os.path.join(HERE, "libpakv_graph.so")


def build_graph_lib() -> str:
    """The HIP-graph step driver (pakv_graph.c) as a shared library."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler for the C client")
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-shared", "-fPIC", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", f"-I{os.path.join(ROOT, 'include')}", GRAPH_SRC, "-o", GRAPH_OUT + ".tmp",
           "-L/opt/rocm/lib", "-lamdhip64", f"-L{PKG}", "-l:libpakv.so",
           "-Wl,-rpath,/opt/rocm/lib", "-Wl,-rpath,$ORIGIN/../../paged_kv_decode_02_amd"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"graph driver build failed:\n{res.stderr}")
    os.replace(GRAPH_OUT + ".tmp", GRAPH_OUT)
    return GRAPH_OUT


def build() -> str:
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler for the C client")
    if not os.path.exists(os.path.join(PKG, "libpakv.so")):
        raise RuntimeError("libpakv.so is not built")
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", f"-I{os.path.join(ROOT, 'include')}", SRC, "-o", OUT + ".tmp",
           "-L/opt/rocm/lib", "-lamdhip64", f"-L{PKG}", "-l:libpakv.so", "-lm",
           "-Wl,-rpath,/opt/rocm/lib", "-Wl,-rpath,$ORIGIN/../../paged_kv_decode_02_amd"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"C client build failed:\n{res.stderr}")
    os.replace(OUT + ".tmp", OUT)
    build_graph_lib()
    return OUT


if __name__ == "__main__":
    print(build())
    sys.exit(0)
