"""Sanitizer builds of the host C / C++ code (CPU only): the oracle (oracle/oracle.c) and the
plan builder (csrc/plan.cpp) are compiled with AddressSanitizer and UndefinedBehaviorSanitizer
(any report is fatal) and driven through every entry point: the oracle on small problems in
every mode, including malformed cu_seqlens and out-of-range gather indices; the plan builder by
a seeded fuzz of 200000 descriptors around and beyond the validation limits."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _build_and_run(tmp_path, compiler, sources, extra, name):
    exe = str(tmp_path / name)
    cmd = [compiler] + SAN + extra + sources + ["-o", exe, "-lm", "-pthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    out = _build_and_run(tmp_path, "gcc", [os.path.join(ROOT, "oracle", "oracle.c"),
                                           os.path.join(HERE, "oracle_drive.c")],
                         ["-std=c11", "-D_GNU_SOURCE", "-ffp-contract=off"], "oracle_drive")
    assert "oracle drive ok" in out


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_plan_builder_under_asan_ubsan(tmp_path):
    out = _build_and_run(tmp_path, "g++", [os.path.join(ROOT, "gemm_epilogue_persistent_amd", "csrc", "plan.cpp"),
                                           os.path.join(HERE, "plan_fuzz.cpp")], ["-std=c++17"], "plan_fuzz")
    assert "plans accepted" in out
