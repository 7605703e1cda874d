"""The library's host side (plan creation, argument validation, workspace
layout and launch descriptors) built from its own source with
AddressSanitizer and UndefinedBehaviorSanitizer and run without a GPU
against launcher stubs that check every descriptor
(tests/host_check/plan_check.cpp)."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM_INCLUDE = "/opt/rocm/include"


def test_plan_and_descriptors_under_sanitizers(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None or not os.path.isdir(ROCM_INCLUDE):
        pytest.skip("needs g++ and the HIP headers")
    exe = tmp_path / "plan_check"
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-D__align__(n)=__attribute__((aligned(n)))",
           "-DHIP_SYMBOL(x)=x",
           f"-I{ROCM_INCLUDE}", f"-I{ROOT}/include", f"-I{ROOT}/orthogonalized_updates_amd/csrc",
           "-x", "c++", f"{ROOT}/orthogonalized_updates_amd/csrc/muonh_abi.hip",
           "-x", "c++", f"{ROOT}/tests/host_check/plan_check.cpp", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    assert "host check ok" in r.stdout


@pytest.mark.parametrize("old,new", [
    # the matrix block one s x s buffer short: the polynomial's output leaves it
    ("G.mat_bytes = nx * xs + 2 * ss;", "G.mat_bytes = nx * xs + ss;"),
    # one apply tile per matrix dropped from the descriptors
    ("q.tiles_per_mat = ts * tl;\n      q.offE = q.fold ? -1 : xin;",
     "q.tiles_per_mat = ts * tl - 1;\n      q.offE = q.fold ? -1 : xin;"),
    # the apply writing the buffer it reads
    ("const int64_t xin = G.offXs[src], xout = G.offXs[1 - src];",
     "const int64_t xin = G.offXs[src], xout = G.offXs[src];"),
])
def test_planted_descriptor_mistakes_are_caught(tmp_path, old, new):
    cxx = shutil.which("g++")
    if cxx is None or not os.path.isdir(ROCM_INCLUDE):
        pytest.skip("needs g++ and the HIP headers")
    src = open(f"{ROOT}/orthogonalized_updates_amd/csrc/muonh_abi.hip").read()
    assert src.count(old) == 1
    bad = tmp_path / "muonh_abi_planted.cc"
    bad.write_text(src.replace(old, new).replace('#include "../../include/muonh.h"',
                                                 '#include "muonh.h"'))
    exe = tmp_path / "plan_check"
    cmd = [cxx, "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__",
           "-D__align__(n)=__attribute__((aligned(n)))", "-DHIP_SYMBOL(x)=x",
           f"-I{ROCM_INCLUDE}", f"-I{ROOT}/include", f"-I{ROOT}/orthogonalized_updates_amd/csrc",
           str(bad), f"{ROOT}/tests/host_check/plan_check.cpp", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode != 0 and "FAIL" in r.stdout
