"""The C ABI's host-side argument checks under AddressSanitizer and
UndefinedBehaviorSanitizer: tests/abi_host_check.cpp calls every entry point
with arguments that are rejected on the host (or an empty batch), built
together with the library's sources with both sanitizers on the host code
only (the device code is built as usual), and must report no failed check
and no sanitizer error.  CPU only: nothing reaches a GPU."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "speculative_decoding_tree_amd", "csrc")
SOURCES = ["api.hip", "verify.hip", "commit.hip", "storeall.hip", "budget.hip", "attention.hip"]


def test_host_checks_under_asan_and_ubsan():
    hipcc = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")
    if not hipcc:
        pytest.skip("hipcc not available")
    tmp = tempfile.mkdtemp(prefix="gdn_asan_")
    try:
        exe = os.path.join(tmp, "abi_host_check")
        cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-I", os.path.join(ROOT, "include"),
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
               "-Wno-unused-command-line-argument"] + [os.path.join(CSRC, s) for s in SOURCES] + \
              [os.path.join(ROOT, "tests", "abi_host_check.cpp"), "-o", exe]
        build = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
        assert build.returncode == 0, build.stderr[-3000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
                   HIP_VISIBLE_DEVICES="")
        run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
        out = run.stdout + run.stderr
        assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
        assert run.returncode == 0 and "0 failures" in run.stdout, out[-3000:]
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
