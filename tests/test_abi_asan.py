"""The C ABI layer (api.cpp, workspace.cpp) built for the host with
AddressSanitizer and UndefinedBehaviorSanitizer, its kernel launchers
replaced by recording stubs (tests/abi_host/stub_launchers.cpp), and driven
through every entry point with exactly sized host arrays
(tests/abi_host/driver.cpp). Needs no GPU: only host code is built (g++)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sequence_parallelism_ulysses_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "abi_host")
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs g++ and the ROCm headers")
def test_abi_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_asan")
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include", f"-I{CSRC}",
           f"-I{ROCM_INCLUDE}", os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "workspace.cpp"),
           os.path.join(HOST, "stub_launchers.cpp"), os.path.join(HOST, "driver.cpp"), "-o", exe, "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert r.stdout.startswith("ok "), r.stdout
    assert "Sanitizer" not in r.stderr, r.stderr[-4000:]
