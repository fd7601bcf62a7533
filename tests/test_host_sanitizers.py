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


def test_sanitizer_catches_planted_overflow(san_libs, tmp_path):
    """The sanitizer run itself is pinned: a copy of the oracle whose P.V loop
    runs one row too far (writing past O and reading past P on the last
    head) must make the same child run fail with an AddressSanitizer
    report."""
    fa_lib, _ = san_libs
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    good = "for (long i = 0; i < N; ++i)\n            weighted_sum(P + i * N, vh, N, d, oh + i * d);"
    assert src.count(good) == 1
    bad_c = tmp_path / "oracle_overflow.c"
    bad_c.write_text(src.replace(good, good.replace("i < N", "i <= N")))
    bad_lib = str(tmp_path / "liboracle_overflow.so")
    subprocess.run(["gcc", *SAN, "-std=c11", "-shared", "-fPIC", "-fopenmp", str(bad_c),
                    "-o", bad_lib, "-lm"], check=True, capture_output=True, text=True)
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": f"{_runtime('libasan.so')}:{_runtime('libubsan.so')}",
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "SAN_FA_LIB": fa_lib, "SAN_ORACLE_LIB": bad_lib, "OMP_NUM_THREADS": "2",
        "PYTHONPATH": ROOT + os.pathsep + env.get("PYTHONPATH", ""),
    })
    # -s: the report goes to the child's stderr, which pytest's own capture
    # would swallow when the sanitizer aborts the process
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
           "-p", "tests.sanitize.plugin", "-m", "not gpu",
           os.path.join(ROOT, "tests", "test_oracle_pins.py")]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode != 0, out[-4000:]
    assert "ERROR: AddressSanitizer" in out, out[-4000:]
