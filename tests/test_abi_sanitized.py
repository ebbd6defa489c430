"""The C ABI's host code (api.cpp) built for the host alone with AddressSanitizer and
UndefinedBehaviorSanitizer, and driven through its argument checks and host
computations (tests/host_checks/abi_checks.cpp). The kernel launchers are stubs
that abort, so the run also shows that every checked call returns before a launch.
No GPU is involved: g++ compiles api.cpp against the HIP headers."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_checks")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(os.path.join(ROCM, "include", "hip")),
                    reason="needs g++ and the HIP headers")
def test_argument_checks_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_checks")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{ROOT}/include",
           f"-I{ROOT}/attention_yarn_rope_amd/csrc",
           os.path.join(ROOT, "attention_yarn_rope_amd", "csrc", "api.cpp"),
           os.path.join(HERE, "launch_stubs.cpp"), os.path.join(HERE, "abi_checks.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, "host build failed:\n" + r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "all argument checks behaved as documented" in out
