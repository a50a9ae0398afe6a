"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two programs are built with gcc / g++ -fsanitize=address,undefined (no
recovery: the first report ends the run with a non-zero status) and run:

  tests/c/oracle_sanitize.c  + oracle/wq_oracle.c: every oracle routine over
      the tested shapes and edge values;
  tests/c/abi_sanitize.cpp   + the library's host ABI layer (wq_abi.cpp) with
      stub launchers: validation, size queries, layout and both planners over
      random tables, on paths that make no HIP runtime call.

Leaks are checked too, except inside the HIP runtime library, which the ABI
program links but never calls.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "weight_only_bit_block_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _env(tmp):
    supp = os.path.join(tmp, "lsan.supp")
    with open(supp, "w") as f:
        f.write("leak:libamdhip64\nleak:libhsa-runtime64\nleak:libdrm\n")
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "abort_on_error=0:halt_on_error=1:detect_leaks=1"
    env["LSAN_OPTIONS"] = f"suppressions={supp}"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "4"
    return env


def _run(cmd, env, timeout):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    return r.returncode, r.stdout + r.stderr


@pytest.fixture(scope="module")
def tmp(tmp_path_factory):
    if shutil.which("gcc") is None or shutil.which("g++") is None:
        pytest.skip("gcc / g++ not available")
    return str(tmp_path_factory.mktemp("sanitize"))


def test_oracle_under_sanitizers(tmp):
    exe = os.path.join(tmp, "oracle_sanitize")
    rc, out = _run(["gcc", "-std=c11", *SAN, "-fopenmp", os.path.join(ROOT, "oracle", "wq_oracle.c"),
                    os.path.join(ROOT, "tests", "c", "oracle_sanitize.c"), "-lm", "-o", exe], None, 300)
    assert rc == 0, out
    rc, out = _run([exe], _env(tmp), 600)
    assert rc == 0 and "all checks passed" in out and "runtime error" not in out, out


def test_abi_host_layer_under_sanitizers(tmp):
    exe = os.path.join(tmp, "abi_sanitize")
    rc, out = _run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I" + os.path.join(ROOT, "include"), os.path.join(CSRC, "wq_abi.cpp"),
                    os.path.join(ROOT, "tests", "c", "abi_sanitize.cpp"),
                    "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe], None, 300)
    assert rc == 0, out
    rc, out = _run([exe], _env(tmp), 300)
    assert rc == 0 and "all checks passed" in out and "runtime error" not in out, out
