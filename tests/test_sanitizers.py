"""CPU sanitizer tier: the oracle's C and libftmoe's host-side workspace arithmetic
(host_layout.hpp: descriptor checks, launch-shape sizing, workspace layouts), each
built with the address and undefined-behaviour sanitizers and run on the host.

tests/sanitize/oracle_check.c drives every oracle entry point on small random
layers; tests/sanitize/host_layout_check.cpp sweeps descriptors, paths and token
counts and checks every workspace region for alignment, size, overlap and end,
and that workspace totals never shrink as tokens grow."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all"]


def _build_and_run(tmp_path, cmd, exe):
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=tmp_path)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=240)
    print(r.stdout[-2000:])
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert r.stdout.strip().endswith("ok")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    exe = tmp_path / "oracle_check"
    cmd = (["gcc", "-std=c11", "-Wno-unknown-pragmas"] + SAN +
           [os.path.join(ROOT, "tests", "sanitize", "oracle_check.c"),
            os.path.join(ROOT, "oracle", "ftmoe_oracle.c"), "-o", str(exe), "-lm"])
    _build_and_run(tmp_path, cmd, exe)


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_workspace_layout_under_address_and_ub_sanitizers(tmp_path):
    exe = tmp_path / "host_layout_check"
    cmd = (["g++", "-std=c++17"] + SAN +
           ["-I", os.path.join(ROOT, "include"),
            "-I", os.path.join(ROOT, "nvfp4_mixture_experts_amd", "csrc"),
            os.path.join(ROOT, "tests", "sanitize", "host_layout_check.cpp"), "-o", str(exe)])
    _build_and_run(tmp_path, cmd, exe)
