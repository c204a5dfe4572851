"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds the library's host code (descriptor validation, plans, workspace
carving, size queries) with the sanitizers on the host side only -- the
gfx950 device code is compiled as usual and never runs -- together with
``tests/host_check/host_check.cpp``, which feeds it about 20,000 fuzzed and
hand-picked descriptors and calls the entry points only with arguments that
must be refused before any launch. No GPU is made visible to the run.
"""
import os
import shutil
import subprocess
import sys

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")
sys.path.insert(0, REPO)
from memory_efficient_long_amd.build import LINK_FLAGS  # noqa: E402

# Each sanitizer flag is preceded by -Xarch_host: host code only.
SANITIZE = ["-Xarch_host", "-fsanitize=address",
            "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(HIPCC is None, reason="hipcc not available")
def test_host_code_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_check")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", *SANITIZE,
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-result",
           "-I", os.path.join(REPO, "include"),
           os.path.join(REPO, "tests", "host_check", "host_check.cpp"),
           os.path.join(REPO, "memory_efficient_long_amd", "csrc", "bpt_layer.hip"), "-o", exe,
           *LINK_FLAGS]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "0 failures" in out and "runtime error" not in out and "ERROR: AddressSanitizer" not in out
    print(out.strip().splitlines()[-1])
