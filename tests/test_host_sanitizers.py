"""The host code of libfo under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The planner (plan.cpp), the partition search (search.cpp) and the C ABI's
argument checks (api.cpp) are compiled by the host compiler with
-fsanitize=address,undefined (every report fatal) into a library of their own,
with the kernel launchers replaced by stand-ins (tests/host_sanitize), and the
planner, search and ABI tests are run against it in a child process with the
sanitizer runtime preloaded.  No GPU code is built or run.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gemm_tile_signaling_amd", "csrc")
OUT_DIR = os.path.join(ROOT, "gemm_tile_signaling_amd", "_build")
LIB = os.path.join(OUT_DIR, "libfo_host_sanitized.so")


def _build():
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not available")
    asan = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not asan or not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("the AddressSanitizer runtime is not available")
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = [os.path.join(CSRC, f) for f in ("plan.cpp", "search.cpp", "api.cpp")]
    srcs.append(os.path.join(ROOT, "tests", "host_sanitize", "launch_stubs.cpp"))
    cmd = [gxx, "-std=c++17", "-shared", "-fPIC", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), *srcs, "-o", LIB,
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return asan


@pytest.mark.slow
def test_planner_search_and_abi_tests_pass_under_sanitizers():
    asan = _build()
    env = dict(os.environ, FO_LIB=LIB, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    tests = ["tests/test_planner_vs_oracle.py", "tests/test_search_vs_oracle.py", "tests/test_abi.py"]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                        *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
    assert " passed" in r.stdout, out
