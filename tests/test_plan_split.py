"""Host check of the tile split of the matrix-core launches (no GPU).

tests/host/plan_split_check.cpp is compiled host-only against the library's ABI
source, with stub kernel launchers, and run: over random ragged batches, every
tile of the Gram, A^2 and product launches is taken by exactly one workgroup,
and each XCD's contiguous range holds about 1/8 of the launch's K slices.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not found")
def test_every_tile_once_and_xcd_work_balanced(tmp_path):
    exe = tmp_path / "plan_split_check"
    build = subprocess.run(
        ["hipcc", "--offload-host-only", "-x", "hip", "-O1", "-std=c++17",
         "-I", os.path.join(ROOT, "include"),
         "-I", os.path.join(ROOT, "newton_schulz_03_amd", "csrc"),
         os.path.join(ROOT, "tests", "host", "plan_split_check.cpp"), "-o", str(exe)],
        capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-3000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0 and run.stdout.startswith("OK"), run.stdout + run.stderr
