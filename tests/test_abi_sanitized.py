"""The library's host code (csrc/pakv.hip: argument checks, sizing, the
decode launch plan) with AddressSanitizer and UBSan on its host side, driven
from C by tests/c_client/abi_fuzz.c: random plans (every (sequence, split)
once, short sequences whole in one item, rotations and item order as stated;
a buffer one word short refused untouched), the sizing calls, every status text, and the argument checks of every entry
point that queues work, with arguments they must refuse (so no kernel is
ever queued). CPU only."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_decode_02_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


@pytest.fixture(scope="module")
def fuzzer(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    gcc, gxx = shutil.which("gcc"), shutil.which("g++")
    if not (os.path.exists(hipcc) and gcc and gxx):
        pytest.skip("hipcc, gcc or g++ is not installed")
    d = tmp_path_factory.mktemp("abi_fuzz")
    lib_o, fuzz_o, exe = str(d / "pakv_host.o"), str(d / "abi_fuzz.o"), str(d / "abi_fuzz")
    steps = [
        # the sanitizers on the host side only (device code is built as usual and never run)
        [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         "-Xarch_host", "-fno-sanitize-recover=all", "-Wno-unused-command-line-argument",
         f"-I{INCLUDE}", f"-I{CSRC}", "-c", os.path.join(CSRC, "pakv.hip"), "-o", lib_o],
        [gcc, "-std=c11", "-O1", "-g", "-Wall", "-Wextra", "-Werror", *SAN, f"-I{INCLUDE}", "-c",
         os.path.join(ROOT, "tests", "c_client", "abi_fuzz.c"), "-o", fuzz_o],
        [gxx, "-fsanitize=address,undefined", fuzz_o, lib_o, "-o", exe, "-L/opt/rocm/lib", "-lamdhip64",
         "-Wl,-rpath,/opt/rocm/lib"],
    ]
    for cmd in steps:
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, f"build failed: {' '.join(cmd)}\n{res.stderr[-4000:]}"
    return exe


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_host_code_under_sanitizers(fuzzer, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([fuzzer, str(seed), "3000"], capture_output=True, text=True, timeout=300, env=env)
    assert res.returncode == 0, f"seed {seed}: exit {res.returncode}\n{res.stdout}\n{res.stderr[-4000:]}"
    assert "ok" in res.stdout
