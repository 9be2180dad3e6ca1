"""The host scheduler (csrc/pakv_sched.cpp) built with AddressSanitizer and
UBSan (g++, host code only) under random operation sequences of
tests/c_client/sched_fuzz.c, which calls every pakv_sched.h entry point,
its error paths included, and checks the block tables and the page
accounting after every operation. CPU only."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FLAGS = ["-O1", "-g", "-Wall", "-Wextra", "-Werror", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", f"-I{os.path.join(ROOT, 'include')}"]


@pytest.fixture(scope="module")
def fuzzer(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not installed")
    d = tmp_path_factory.mktemp("sched_fuzz")
    fuzz_o, sched_o, exe = str(d / "fuzz.o"), str(d / "sched.o"), str(d / "sched_fuzz")
    steps = [
        [gxx, "-x", "c", "-std=c11", *FLAGS, "-c", os.path.join(ROOT, "tests", "c_client", "sched_fuzz.c"),
         "-o", fuzz_o],
        [gxx, "-std=c++17", *FLAGS, "-c", os.path.join(ROOT, "paged_kv_decode_02_amd", "csrc", "pakv_sched.cpp"),
         "-o", sched_o],
        [gxx, "-fsanitize=address,undefined", fuzz_o, sched_o, "-o", exe],
    ]
    for cmd in steps:
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, f"build failed: {' '.join(cmd)}\n{res.stderr}"
    return exe


@pytest.mark.parametrize("seed", [1, 2, 3, 4])   # odd seeds: static batching, even: continuous
def test_scheduler_under_sanitizers(fuzzer, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([fuzzer, str(seed), "20000"], capture_output=True, text=True, timeout=300, env=env)
    assert res.returncode == 0, f"seed {seed}: exit {res.returncode}\n{res.stdout}\n{res.stderr[-4000:]}"
    assert "ok" in res.stdout
