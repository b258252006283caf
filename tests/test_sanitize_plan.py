"""The host plan (csrc/tdp_plan.cpp) built with AddressSanitizer and
UndefinedBehaviorSanitizer (g++, host code only) and driven by random valid
and invalid descriptors (tests/sanitize/plan_fuzz.cpp): no out-of-bounds
access, no undefined behaviour, every invalid descriptor refused with a
status, and the plan's invariants on every valid one.  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def fuzzer(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path_factory.mktemp("sanitize") / "plan_fuzz")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-Wall", "-Wextra", "-Werror",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "sanitize", "plan_fuzz.cpp"),
           os.path.join(ROOT, "tiled_video_diffusion_amd", "csrc", "tdp_plan.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_plan_under_sanitizers(fuzzer, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([fuzzer, "3000", str(seed)], capture_output=True, text=True,
                       timeout=300, env=env)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    ok, valid, invalid = r.stdout.split()[-3:]
    assert ok == "ok" and int(valid) > 500 and int(invalid) > 500, r.stdout
