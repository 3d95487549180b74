"""The C ABI layer (api.hip) built for the host with AddressSanitizer and
UndefinedBehaviorSanitizer, its kernel launchers replaced by recorders
(tests/sanitize/launch_stubs.cpp), and driven through every entry point by
tests/sanitize/abi_host_sanitize.cpp: valid calls checked for what a launch would
receive, invalid ones for their status, host arrays sized exactly, 64-bit size
overflows. No GPU and no HIP runtime are involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_abi_layer_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "abi_sanitize")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.join(ROOT, 'sequence_dit_amd', 'csrc')}", f"-I{SAN}",
           "-x", "c++", os.path.join(ROOT, "sequence_dit_amd", "csrc", "api.hip"),
           "-x", "none", os.path.join(SAN, "launch_stubs.cpp"), os.path.join(SAN, "abi_host_sanitize.cpp"),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and "abi sanitize ok" in r.stdout, (r.stdout + r.stderr)[-4000:]
