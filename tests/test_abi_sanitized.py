"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

api.hip (argument checks and launch set-up) is compiled with the sanitizers on its host side
only and linked with the library's other objects into a driver program
(tests/sanitize/abi_driver.cpp) that calls every entry point's error paths; those return
before any HIP call, so no GPU is needed. The driver must exit 0 with no sanitizer report."""
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "_build")
OUT = os.path.join(BUILD, "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ROCM_LIB = "/opt/rocm/lib"

# sanitizer options for the host compiler only (each after -Xarch_host)
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_abi_error_paths_under_sanitizers():
    others = [o for o in glob.glob(os.path.join(BUILD, "*.hip.o")) if not o.endswith("api.hip.o")]
    if not others:
        pytest.skip("library objects not built (run python -m io_aware_softmax_03_amd.build)")
    os.makedirs(OUT, exist_ok=True)
    api_o = os.path.join(OUT, "api_san.o")
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
          *HOST_SAN, "-c", os.path.join(ROOT, "io_aware_softmax_03_amd", "csrc", "api.hip"), "-o", api_o])
    drv_o = os.path.join(OUT, "abi_driver.o")
    _run(["g++", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"), "-c",
          os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), "-o", drv_o])
    exe = os.path.join(OUT, "abi_driver")
    _run(["g++", "-fsanitize=address,undefined", drv_o, api_o, *sorted(others), f"-L{ROCM_LIB}",
          f"-Wl,-rpath,{ROCM_LIB}", "-lamdhip64", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    report = res.stdout + res.stderr
    assert res.returncode == 0, report
    assert "runtime error" not in report and "AddressSanitizer" not in report, report
    assert "all error paths returned their expected status" in res.stdout
