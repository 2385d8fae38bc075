"""CPU sanitizer tier: the oracle and the C-ABI layer's host code built with
AddressSanitizer and UndefinedBehaviorSanitizer (gcc/g++, host only) and run
once.  The oracle runs every entry point on small seeded inputs (including a
NaN token); the C-ABI layer (include/moe.h over moe_api.hip, compiled as
plain C++ against host stand-ins of the kernel launchers) is driven through
its validation paths: each rejected call must return the documented code and
launch nothing."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None, reason="needs gcc/g++")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r.stdout


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    _run(["gcc", "-std=c11", "-Wall", "-Wno-unknown-pragmas", *SAN, os.path.join(ROOT, "tests/sanitize/oracle_driver.c"),
          os.path.join(ROOT, "oracle/moe_oracle.c"), "-o", exe, "-lm"])
    assert _run([exe], env=ENV).strip() == "ok"


def test_abi_validation_under_sanitizers(tmp_path):
    inc = ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "mixture_experts_ffn_05_amd/csrc"),
           "-I" + os.path.join(ROOT, "include")]
    if not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"):
        pytest.skip("HIP headers not installed")
    objs = []
    for src, lang in (("mixture_experts_ffn_05_amd/csrc/moe_api.hip", "c++"),
                      ("tests/sanitize/stub_launchers.cpp", "c++")):
        o = str(tmp_path / (os.path.basename(src) + ".o"))
        _run(["g++", "-std=c++17", *SAN, *inc, "-c", "-x", lang, os.path.join(ROOT, src), "-o", o])
        objs.append(o)
    o = str(tmp_path / "abi_driver.o")
    _run(["gcc", "-std=c11", *SAN, "-I" + os.path.join(ROOT, "include"), "-c",
          os.path.join(ROOT, "tests/sanitize/abi_driver.c"), "-o", o])
    exe = str(tmp_path / "abi_asan")
    _run(["g++", *SAN, *objs, o, "-o", exe])
    assert _run([exe], env=ENV).strip() == "ok"
