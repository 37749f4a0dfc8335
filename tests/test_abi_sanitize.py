"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): tests/sanitize/abi_sanitize.cpp drives the argument validation of
every entry point, the status strings and the draft-length controller, built
together with the library's sources with host-side sanitizers (device code is
built without them and never runs here)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rejection_sampling_verify_09_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "abi_san")
    srcs = [os.path.join(CSRC, f) for f in ("sv_kernels.hip", "sv_api.hip", "sv_lmhead.hip", "sv_dynk.cpp")]
    srcs.append(os.path.join(ROOT, "tests", "sanitize", "abi_sanitize.cpp"))
    cmd = [HIPCC, "--offload-arch=gfx950", "-O0", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-g",
           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, *srcs, "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert b.returncode == 0, b.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.stdout[-2000:], r.stderr[-3000:])
    shutil.rmtree(tmp_path, ignore_errors=True)
