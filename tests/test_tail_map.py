"""Host logic of the partial-wave split: the workgroup map tile::tail_unit
(built from the kernel header for the host with hipcc and run on the CPU)
takes every whole tile and every split unit exactly once, whole tiles first
on every XCD."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC),
                    reason="hipcc not available")
def test_tail_unit_map(tmp_path):
    exe = tmp_path / "tail_map_check"
    r = subprocess.run([HIPCC, "-O1", "-std=c++17", "-x", "hip", "--offload-arch=gfx950",
                        os.path.join(HERE, "tail_map_check.hip"), "-o", str(exe)],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.startswith("ok "), r.stdout + r.stderr
