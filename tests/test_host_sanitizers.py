"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer: the
oracle (oracle/oracle.c) and the C ABI's argument validation
(csrc/fa_api.cpp with the launch planning of csrc/fa_plan.cpp, its kernel
launchers replaced by host stubs) are compiled by gcc/g++ with
-fsanitize=address,undefined -fno-sanitize-recover=all, and the oracle pins
and the ABI validation tests run against those builds in a child process
(with the sanitizer runtimes preloaded).  Any sanitizer report aborts the
child and fails the test.  GPU code is not built with sanitizers."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_32_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def san_libs(tmp_path_factory):
    if not (_runtime("libasan.so") and _runtime("libubsan.so")):
        pytest.skip("gcc sanitizer runtimes not installed")
    d = tmp_path_factory.mktemp("san")
    fa_lib = str(d / "libfa_hostcheck.so")
    subprocess.run(["g++", *SAN, "-std=c++17", "-shared", "-fPIC", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", "/opt/rocm/include",
                    os.path.join(CSRC, "fa_api.cpp"), os.path.join(CSRC, "fa_plan.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "stub_launchers.cpp"),
                    "-o", fa_lib], check=True, capture_output=True, text=True)
    or_lib = str(d / "liboracle_san.so")
    subprocess.run(["gcc", *SAN, "-std=c11", "-shared", "-fPIC", "-fopenmp",
                    os.path.join(ROOT, "oracle", "oracle.c"), "-o", or_lib, "-lm"],
                   check=True, capture_output=True, text=True)
    return fa_lib, or_lib


def test_pins_and_abi_under_sanitizers(san_libs):
    fa_lib, or_lib = san_libs
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": f"{_runtime('libasan.so')}:{_runtime('libubsan.so')}",
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
        "SAN_FA_LIB": fa_lib, "SAN_ORACLE_LIB": or_lib, "OMP_NUM_THREADS": "4",
        "PYTHONPATH": ROOT + os.pathsep + env.get("PYTHONPATH", ""),
    })
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
           "-p", "tests.sanitize.plugin", "-m", "not gpu",
           os.path.join(ROOT, "tests", "test_abi.py"),
           os.path.join(ROOT, "tests", "test_oracle_pins.py"),
           os.path.join(ROOT, "tests", "test_tiled_model.py")]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    print(out)
    assert r.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
