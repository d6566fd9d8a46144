"""The C-ABI validation layer (csrc/abi.cpp) built for the host with
AddressSanitizer and UBSan, driven through every validation branch by
tests/sanitize/abi_cases.cpp.  The launchers and size functions are host-only
stand-ins (tests/sanitize/abi_stubs.cpp), so this needs no GPU: it checks
that argument validation reads only what the header says it reads (host
offsets of exactly n_docs + 1 entries), has no undefined behaviour on extreme
sizes, and returns the documented status with a message."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the HIP headers")
def test_abi_validation_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_cases")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "attention_target_amd", "csrc"),
           "-I", SAN, os.path.join(ROOT, "attention_target_amd", "csrc", "abi.cpp"),
           os.path.join(SAN, "abi_stubs.cpp"), os.path.join(SAN, "abi_cases.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    assert "cases passed" in r.stdout, r.stdout
