"""The C ABI's host code under AddressSanitizer (CPU only).

The library (every translation unit of it) is built with the sanitizer on its
host code only (the device code is compiled as usual, without it; the per-unit
scheduling flags do not matter here), and a small C++ program
(`abi_host_asan.cpp`, built with the same compiler and sanitizer runtime)
drives every entry point's argument validation and the built-in table over a
grid of shapes.  No call reaches a launch, so no GPU is needed; a sanitizer
report or an unexpected return code fails the test.
"""
import os
import shutil
import subprocess

import pytest

from moe_gate_up_amd.build import SOURCES   # every translation unit of the library

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                                reason="needs ROCm's hipcc and clang++")


def test_host_code_under_address_sanitizer(tmp_path):
    lib = tmp_path / "libmoe_decode_asan.so"
    exe = tmp_path / "abi_host_asan"
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "moe_gate_up_amd", "csrc")]
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", *inc,
                    *[os.path.join(ROOT, "moe_gate_up_amd", "csrc", src) for src, _ in SOURCES], "-o", str(lib)],
                   check=True, capture_output=True, timeout=600)
    subprocess.run([CLANG, "-O1", "-g", "-std=c++17", "-fsanitize=address", "-fno-omit-frame-pointer",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "abi_host_asan.cpp"),
                    str(lib), f"-Wl,-rpath,{tmp_path}", "-o", str(exe)],
                   check=True, capture_output=True, timeout=600)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=99")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "0 failures" in r.stdout
