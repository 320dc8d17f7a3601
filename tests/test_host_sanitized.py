"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

`tests/host_checks.cpp` drives every entry point through argument validation,
workspace sizing, the per-thread error text and (on a host without a GPU) the
launch and allocation failure paths.  The ABI layer (`csrc/api.hip`) is rebuilt
here with the sanitizers on its host code only; the kernels come from the built
library.  Any sanitizer report or failed check fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "parallax_local_linear_amd")
LIB = os.path.join(PKG, "libparallax.so")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")

# host-only sanitizer flags: each one behind -Xarch_host so no device code is instrumented
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined"]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    if not os.path.exists(LIB):
        pytest.skip("libparallax.so not built")
    d = tmp_path_factory.mktemp("host_san")
    inc = ["-I", os.path.join(ROOT, "include")]
    api_o, drv_o, exe = str(d / "api.o"), str(d / "host_checks.o"), str(d / "host_checks")
    steps = [
        [HIPCC, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "--cuda-host-only", *SAN,
         *inc, "-c", os.path.join(PKG, "csrc", "api.hip"), "-o", api_o],
        [HIPCC, "-O1", "-g", "-std=c++17", *SAN, *inc, "-D__HIP_PLATFORM_AMD__",
         "-I", os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "include"), "-x", "c++", "-c",
         os.path.join(ROOT, "tests", "host_checks.cpp"), "-o", drv_o],
        [HIPCC, *SAN, drv_o, api_o, LIB, "-Wl,-rpath," + PKG, "-o", exe],
    ]
    for cmd in steps:
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stdout + res.stderr
    return exe


def test_host_code_under_sanitizers(driver):
    env = dict(os.environ)
    # the HIP runtime keeps allocations for the life of the process
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    res = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=120)
    out = res.stdout + res.stderr
    assert "ERROR: AddressSanitizer" not in out, out
    assert "runtime error:" not in out, out
    assert res.returncode == 0, out
    assert "0 failed" in res.stdout, out
