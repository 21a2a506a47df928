"""The host C++ of the C-ABI layer (api.cpp: contract and shape validation,
workspace sizing; contract.cpp: the contract JSON, its digests and SHA-256)
built with AddressSanitizer and UndefinedBehaviorSanitizer by g++, and run
by a C++ driver (tests/host_sanitize/driver.cpp) that makes the calls of
test_abi.py and test_contract_identity.py -- every rejection path of every
entry point, empty calls, workspace queries, the JSON at every short buffer
size, the digests and SHA-256 over every length up to 300 bytes -- in an
instrumented process. The kernel launchers are replaced by stand-ins that
fail, so no call reaches a GPU. No GPU code is built here.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "split_invariant_deterministic_amd", "csrc")
HS = os.path.join(ROOT, "tests", "host_sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "include")),
                                reason="needs g++ and the ROCm headers")


def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "host_sanitize")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{ROOT}/include",
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "contract.cpp"), os.path.join(HS, "stubs.cpp"),
           os.path.join(HS, "driver.cpp"), "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
    assert r.stdout.startswith("host checks passed: ")
    assert int(r.stdout.split(":")[1]) > 400
