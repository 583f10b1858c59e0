"""Host checks of csrc/ra_plan.h that the C ABI does not expose: the order in
which workgroups are spread over the 8 XCDs (a bijection; balanced causal
work per XCD; a head's tiles on as few XCDs as the grid allows)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sequence_transformer_attention_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs a host C++ compiler")
def test_xcd_remap(tmp_path):
    exe = tmp_path / "plan_check"
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", CSRC, os.path.join(ROOT, "tests", "plan_check.cpp"),
                    "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout + out.stderr


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None, reason="needs host compilers")
def test_kernel_walk_and_mask_decisions_match_the_oracle(tmp_path):
    """The tile walk, mask flags and visible prefixes the kernels take
    (csrc/ra_plan.h, composed as the kernels compose them) against the
    oracle's classifier and visible-pair count, bit for bit."""
    obj = tmp_path / "ra_oracle.o"
    subprocess.run(["gcc", "-std=c11", "-O2", "-c", os.path.join(ROOT, "oracle", "ra_oracle.c"), "-o", str(obj)],
                   check=True)
    exe = tmp_path / "walk_check"
    subprocess.run(["g++", "-std=c++17", "-O2", "-I", CSRC, os.path.join(ROOT, "tests", "walk_check.cpp"), str(obj),
                    "-lpthread", "-lm", "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0 and out.stdout.startswith("ok"), out.stdout + out.stderr
