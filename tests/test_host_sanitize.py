"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is compiled with both sanitizers on its host code (-Xarch_host;
the device code is built as usual), and tests/host_sanitize/abi_errors.cpp
drives every entry point's
argument errors, the workspace-size functions and the host RoPE table builders
through it.  Compute calls all carry an argument error, so nothing reaches a
GPU; any out-of-bounds host access or undefined behaviour on those paths aborts
the driver."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_attention_diffusion_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_sanitize")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain missing")
def test_abi_error_paths_under_asan_and_ubsan(tmp_path):
    lib = tmp_path / "libsana_linattn_host_san.so"
    san = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined"]
    host_san = [flag for f in san for flag in ("-Xarch_host", f)]
    build_lib = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
                 "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                 os.path.join(CSRC, "sana_linattn.hip"), "-o", str(lib)]
    r = subprocess.run(build_lib, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = tmp_path / "abi_errors"
    build_exe = [CLANG, "-O1", "-g", "-std=c++17", *san, "-I", os.path.join(ROOT, "include"),
                 os.path.join(HERE, "abi_errors.cpp"), "-L", str(tmp_path), "-lsana_linattn_host_san",
                 f"-Wl,-rpath,{tmp_path}", "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", str(exe)]
    r = subprocess.run(build_exe, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "all ABI error paths behaved" in r.stdout
