"""Host sanitizer builds (CPU only): the C oracle under gcc's AddressSanitizer and
UndefinedBehaviorSanitizer, and the host half of the C ABI (ssm_api.hip compiled host-only with
hipcc, the same sanitizers) linked with stand-ins for the kernel launchers that check every
region a launch would touch against the state layout. Both drivers live in tests/native/; a
sanitizer report, a failed check or a non-zero exit fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
OUT = os.path.join(ROOT, "tests", "native", "_build")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")


def _run(cmd, timeout):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout, env=ENV)
    return r.returncode, r.stdout + r.stderr


def test_oracle_under_asan_ubsan():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_sanitize")
    rc, log = _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fopenmp",
                    os.path.join(ROOT, "oracle", "ssm_oracle.c"),
                    os.path.join(NATIVE, "oracle_sanitize_main.c"), "-lm", "-o", exe], 300)
    assert rc == 0, log[-4000:]
    rc, log = _run([exe], 300)
    assert rc == 0 and "0 failures" in log and "Sanitizer" not in log, log[-4000:]


def test_abi_host_half_under_asan_ubsan():
    hipcc = "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "abi_host_sanitize")
    srcs = [os.path.join(ROOT, "ssm_decode_state_amd", "csrc", "ssm_api.hip"),
            os.path.join(NATIVE, "abi_host_stubs.cpp"), os.path.join(NATIVE, "abi_host_main.cpp")]
    cmd = [hipcc, "-x", "hip", "--offload-host-only", "-std=c++17", "-O1", "-g",
           "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
           "-fsanitize=undefined", "-fno-sanitize-recover=all",
           "-I" + os.path.join(ROOT, "include")] + srcs + ["-o", exe]
    rc, log = _run(cmd, 600)
    assert rc == 0, log[-4000:]
    rc, log = _run([exe], 300)
    assert rc == 0 and "host ABI sanitizer run" in log and "Sanitizer" not in log, log[-4000:]
