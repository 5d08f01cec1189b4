"""The C ABI's host code under AddressSanitizer and UBSan (CPU only).

tests/host/sweep.cpp drives every entry point -- the workspace planners over
a grid of batch, block, head, dim and length sizes, valid calls and invalid
ones -- against capi.hip built for the host only with the sanitizers, the
kernel launches replaced by tests/host/stubs.hip (which checks each plan it
receives and launches nothing). Device code is not built.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_c_abi_host_paths_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "sweep")
    cmd = [HIPCC, "--offload-arch=gfx950", "--offload-host-only", "-O1", "-g",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "verify_attention_amd", "csrc"),
           os.path.join(ROOT, "verify_attention_amd", "csrc", "capi.hip"),
           os.path.join(ROOT, "tests", "host", "stubs.hip"),
           "-x", "c++", os.path.join(ROOT, "tests", "host", "sweep.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    assert "sweep ok" in r.stdout
