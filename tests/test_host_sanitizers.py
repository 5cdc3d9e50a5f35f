"""libkvq's host code (kvq_api.cpp: argument validation of every entry point;
kvq_host.cpp: Lloyd-Max tables, seeded signs, sizes, status strings) built
with g++ under AddressSanitizer and UndefinedBehaviorSanitizer and driven by
tests/native/host_sanitize.cpp, with the kernel launches stubbed out (CPU, no
GPU): every check must pass and neither sanitizer may report anything."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "compressed_decode_attention_randomized_amd", "csrc")
HIP_INCLUDE = "/opt/rocm/include"


def test_host_code_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(HIP_INCLUDE):
        pytest.skip("g++ or the HIP headers are not available")
    exe = str(tmp_path / "kvq_host_sanitize")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-static-libasan",
           "-D__HIP_PLATFORM_AMD__", "-I", HIP_INCLUDE, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "kvq_api.cpp"), os.path.join(CSRC, "kvq_host.cpp"),
           os.path.join(ROOT, "tests", "native", "host_sanitize.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, f"build failed:\n{r.stderr[-4000:]}"
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "host checks passed" in r.stdout
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
