"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): tests/sanitize/host_checks.cpp drives the argument checks, the
tile-map cache and host builders, the split choice, the workspace and scratch
sizing and the lane-mask table, with host stand-ins for the HIP runtime and the
device launchers (see that file).  Built with the host compiler; no device code
is compiled with a sanitizer."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dit_circular_local_amd", "csrc")


@pytest.mark.slow
def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = os.path.join(str(tmp_path), "host_checks")
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "clear_attn.cpp"), os.path.join(CSRC, "tilemap_host.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert run.returncode == 0, run.stderr[-4000:]
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr
    assert "host checks passed" in run.stdout
