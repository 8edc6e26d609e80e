"""Host-side code under the address and undefined-behaviour sanitizers (CPU only, no GPU).

* tests/host/test_plan.cpp: the planner's attention grid against the device's placement rule
  (restated as the prep kernels compute it, on both sides of the longest-first user limit), the
  workspace layouts and the batch checks; built with g++ -fsanitize=address,undefined.
* tests/test_abi_cpu.py run again against the host-sanitized build of the library
  (python -m generative_recommendation_ranking_amd.build --sanitize), with the ASan runtime
  preloaded.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "generative_recommendation_ranking_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_planner_under_sanitizers(tmp_path):
    exe = str(tmp_path / "test_plan")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           "-fno-sanitize-recover=undefined", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "host", "test_plan.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "planner checks passed" in r.stdout


def test_abi_checks_under_sanitizers():
    from generative_recommendation_ranking_amd import build as B
    try:
        B.hipcc()
    except RuntimeError:
        pytest.skip("needs hipcc")
    lib = B.build_library(sanitize=True)
    env = dict(os.environ, MTGR_LIB=lib, LD_PRELOAD=B.sanitizer_runtime(), ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
