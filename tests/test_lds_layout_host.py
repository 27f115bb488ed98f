"""The prefill kernel's LDS layouts, checked on the host (no GPU).

tests/lds_layout_check.cpp includes the kernel's own layout header
(gated_delta_rule_10_amd/csrc/kda_pipe_layout.h) and checks that each layout is
a bijection onto its buffer, that the per-lane offsets the kernel steps through
(one XOR per unrolled index) equal the layout functions -- so the producers
write exactly where the consumers read -- and that every access has conflict
degree 1 under the bank rules the header states (measured on gfx950 with
single-instruction patterns).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs a host C++ compiler")
def test_lds_layouts(tmp_path):
    exe = tmp_path / "lds_layout_check"
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", os.path.join(ROOT, "gated_delta_rule_10_amd", "csrc"),
                    os.path.join(ROOT, "tests", "lds_layout_check.cpp"), "-o", str(exe)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.strip().endswith("ok"), res.stdout
