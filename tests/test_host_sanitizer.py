"""The C ABI's argument validation and workspace planning under host
AddressSanitizer and UndefinedBehaviorSanitizer (CPU only, no launch).

wukong_abi.cpp is compiled with both sanitizers on its host code only (the
device side of the file, the static workspace array of the no-allocation
entry point, is compiled as usual), linked with a C driver that calls every
size query and a set of calls the library must reject before launching, and
resolved against libwukong.so for the kernel launchers it never reaches.
A sanitizer report or a failed expectation fails the test."""
import os
import shutil
import subprocess

import pytest

import recommender_feature_interaction_amd as wk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "recommender_feature_interaction_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "host_sanitizer")
HIPCC = "/opt/rocm/bin/hipcc"

pytestmark = [
    pytest.mark.skipif(not os.path.exists(wk.library_path()), reason="libwukong.so not built"),
    pytest.mark.skipif(not os.path.exists(HIPCC) or shutil.which("gcc") is None, reason="needs hipcc and gcc"),
]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0 or kw.get("check") is False, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.timeout(600)
def test_validation_and_planning_under_asan_and_ubsan():
    os.makedirs(OUT, exist_ok=True)
    inc = [f"-I{CSRC}", f"-I{os.path.join(ROOT, 'include')}"]
    abi_o = os.path.join(OUT, "wukong_abi_san.o")
    # host-side sanitizers only: every -fsanitize flag goes to the host compilation
    _run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
          "-Wno-unused-command-line-argument", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          *inc, "-c", os.path.join(CSRC, "wukong_abi.cpp"), "-o", abi_o])
    drv_o = os.path.join(OUT, "abi_validation.o")
    _run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", *inc[1:], "-c",
          os.path.join(ROOT, "tests", "host_sanitizer", "abi_validation.c"), "-o", drv_o])
    exe = os.path.join(OUT, "abi_validation")
    libdir = os.path.dirname(wk.library_path())
    # the hipcc-built object is clang code: link with clang's sanitizer runtimes
    _run([HIPCC, "-fuse-ld=lld", drv_o, abi_o, "-o", exe, "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined", f"-L{libdir}", "-lwukong", f"-Wl,-rpath,{libdir}",
          "-Wno-unused-command-line-argument"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "all expectations met" in r.stdout
