"""The C ABI used from plain C (CPU only): tests/c/abi_smoke.c is compiled
against include/kda.h alone, linked against the built libkda.so and run; it
exercises the argument checks of every entry point, none of which reaches
the GPU."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_plain_c_program(tmp_path):
    import gated_delta_rule_61_amd as kda
    if not os.path.exists(kda.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    exe = tmp_path / "abi_smoke"
    libdir = os.path.dirname(kda.LIB_PATH)
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                           os.path.join(ROOT, "tests", "c", "abi_smoke.c"), "-L", libdir, "-lkda",
                           f"-Wl,-rpath,{libdir}", "-o", str(exe)])
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "kda C ABI ok" in r.stdout
