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
