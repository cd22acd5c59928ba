"""The host-side C code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only; no device code is built here):

- the C ABI layer (csrc/ssd_api.cpp: every argument check, the argument
  blocks handed to the kernel launchers, and the debug-build check that the
  slot_idx entries of a call are distinct), driven by tests/native/
  abi_host_check.cpp against stand-ins for the launchers;
- the fp64 oracle (oracle/ssd_oracle.c), driven by tests/native/
  oracle_check.c (varlen pack with empty and chunk-multiple sequences, every
  optional output, a closed-form case, the argument checks).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
CSRC = os.path.join(ROOT, "exact_replay_decode_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _build_and_run(tmp_path, compiler, sources, flags, name):
    exe = str(tmp_path / name)
    r = subprocess.run([compiler, *SAN, *flags, *sources, "-o", exe], capture_output=True,
                       text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    return r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_abi_layer_under_sanitizers(tmp_path):
    out = _build_and_run(
        tmp_path, "g++",
        [os.path.join(CSRC, "ssd_api.cpp"), os.path.join(NATIVE, "abi_host_check.cpp")],
        ["-std=c++17", "-DSSD_DEBUG_CHECKS", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC], "abi_host_check")
    assert "0 failed expectations" in out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    out = _build_and_run(
        tmp_path, "gcc",
        [os.path.join(ROOT, "oracle", "ssd_oracle.c"), os.path.join(NATIVE, "oracle_check.c")],
        ["-std=c11", "-fopenmp", "-ffp-contract=off", "-lm"], "oracle_check")
    assert "0 failed expectations" in out
