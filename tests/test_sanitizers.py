"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code
(CPU only): the fp64 oracle (oracle/kda_oracle.c, with OpenMP) and the C
ABI's validation and launch planning (kda_abi.hip compiled as plain C++ with
stub kernel launchers, tests/sanitize/abi_main.cpp).  Each driver exercises
every entry point on small inputs, including empty and one-token sequences,
and exits 0 only if its own checks pass; any sanitizer report aborts it
(-fno-sanitize-recover=all)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2")


def _build_and_run(cmd, exe):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0 and "asan" in (res.stderr or "").lower() and "cannot find" in res.stderr:
        pytest.skip("sanitizer runtime not installed: " + res.stderr.strip()[:200])
    assert res.returncode == 0, res.stderr
    run = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
    return out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    cmd = ["gcc", "-std=c99", *SAN, "-fopenmp", "-o", exe,
           os.path.join(ROOT, "tests", "sanitize", "oracle_main.c"),
           os.path.join(ROOT, "oracle", "kda_oracle.c"), "-lm"]
    assert "all checks passed" in _build_and_run(cmd, exe)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the HIP headers not available")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_san")
    cmd = ["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "gated_delta_rule_amd", "csrc"),
           "-x", "c++", os.path.join(ROOT, "gated_delta_rule_amd", "csrc", "kda_abi.hip"),
           "-x", "c++", os.path.join(ROOT, "tests", "sanitize", "abi_main.cpp"), "-o", exe]
    assert "all checks passed" in _build_and_run(cmd, exe)
