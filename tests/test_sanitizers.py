"""CPU runs under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU):

* the host side of the HIP library (argument checks, workspace sizing, error
  strings of every entry point), built with both sanitizers on the host code
  and driven by the plain-C program tests/c/abi_smoke.c;
* the fp64 oracle (every entry point and variant, OpenMP on), driven by
  tests/c/oracle_smoke.c.
Any sanitizer report makes the program exit nonzero."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def test_oracle_under_sanitizers(tmp_path):
    exe = tmp_path / "oracle_smoke"
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c99", "-Wall", "-Werror", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-fopenmp",
                           os.path.join(ROOT, "tests", "c", "oracle_smoke.c"),
                           os.path.join(ROOT, "oracle", "kda_oracle.c"), "-lm", "-o", str(exe)])
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=ENV)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle C smoke ok" in r.stdout


def test_host_library_under_sanitizers(tmp_path):
    clang = "/opt/rocm/llvm/bin/clang"
    if not os.path.exists(clang) or shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("ROCm clang / hipcc not available")
    from gated_delta_rule_61_amd import _build
    lib = _build.build_sanitized(str(tmp_path / "asan"))
    libdir = os.path.dirname(lib)
    exe = tmp_path / "abi_smoke"
    subprocess.check_call([clang, "-std=c99", "-Wall", "-Werror", "-g", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
                           os.path.join(ROOT, "tests", "c", "abi_smoke.c"), "-L", libdir, "-lkda",
                           f"-Wl,-rpath,{libdir}", "-o", str(exe)])
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=ENV)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "kda C ABI ok" in r.stdout
