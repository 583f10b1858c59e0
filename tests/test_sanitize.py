"""The oracle and the library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

  * oracle/ra_oracle.c with gcc -fsanitize=address,undefined, driven by
    tests/sanitize_oracle.c through every entry point on small inputs;
  * the library's host code (argument validation, planner queries) with the
    sanitizers on the host side of the hipcc build only (a shared library),
    driven by tests/sanitize_abi.cpp with fake device addresses that every
    call rejects before touching the HIP runtime.
Any sanitizer report aborts the driver (no recovery), failing the test.
"""
import os
import shutil
import subprocess

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sequence_transformer_attention_amd", "csrc")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
CLANG = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib", "llvm", "bin", "clang++")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "sanitize_oracle"
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "ra_oracle.c"),
                    os.path.join(ROOT, "tests", "sanitize_oracle.c"), "-lpthread", "-lm", "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, env=ENV, timeout=600)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout + out.stderr


# fake device addresses: never where a GPU could be reached
@pytest.mark.skipif(torch.cuda.is_available() or not os.path.exists(HIPCC) or not os.path.exists(CLANG),
                    reason="CPU-only, needs hipcc")
def test_library_host_code_under_asan_and_ubsan(tmp_path):
    lib = tmp_path / "libringattn_san.so"
    srcs = [os.path.join(CSRC, f) for f in ("ra_api.cpp", "ra_kernels.hip", "ra_f32.hip", "ra_bwd.hip", "ra_state.hip")]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form"] + san + \
          ["-x", "hip"] + srcs + ["-o", str(lib)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    exe = tmp_path / "sanitize_abi"
    res = subprocess.run([CLANG, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                          "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "sanitize_abi.cpp"),
                          str(lib), f"-Wl,-rpath,{tmp_path}", "-o", str(exe)], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True, env=ENV, timeout=600)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout + out.stderr[-4000:]
