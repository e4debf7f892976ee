"""Host check of the tile split of the matrix-core launches (no GPU).

tests/host/plan_split_check.cpp is compiled host-only against the library's ABI
source, with stub kernel launchers, and run: over random ragged batches, every
tile of the Gram, A^2 and product launches is taken by exactly one workgroup,
each XCD's contiguous range holds about 1/8 of the launch's K slices, and the
run-time claims (per-XCD pools, or a ragged launch's single queue) hand out
every pool tile once.  Copies of the source with planted mistakes in the
planner must make the check fail.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "newton_schulz_03_amd", "csrc")


def _check(tmp_path, csrc):
    exe = tmp_path / "plan_split_check"
    build = subprocess.run(
        ["hipcc", "--offload-host-only", "-x", "hip", "-O1", "-std=c++17",
         "-I", os.path.join(ROOT, "include"), "-I", str(csrc),
         os.path.join(ROOT, "tests", "host", "plan_split_check.cpp"), "-o", str(exe)],
        capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-3000:]
    return subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not found")
def test_every_tile_once_and_xcd_work_balanced(tmp_path):
    run = _check(tmp_path, CSRC)
    assert run.returncode == 0 and run.stdout.startswith("OK"), run.stdout + run.stderr


# (text in muon_abi.hip, its replacement, the failure the check must report)
PLANTED = [
    ("    std::sort(q.begin(), q.end());",
     "    std::sort(q.begin(), q.end()); std::reverse(q.begin(), q.end());",
     "queue not longest first"),
    ("  if (queue && ragged && q.size() <= static_cast<size_t>(kOrderCap)) {",
     "  if (queue && q.size() <= static_cast<size_t>(kOrderCap)) {",
     "single queue chosen wrongly"),
    ("  sp.grid = static_cast<int32_t>((longest + pool) * kXcd);",
     "  sp.grid = static_cast<int32_t>((longest + pool / 2) * kXcd);",
     "grid is not 8 x (longest range + pool)"),
]


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not found")
@pytest.mark.parametrize("old,new,failure", PLANTED)
def test_planted_planner_mistakes_fail(tmp_path, old, new, failure):
    csrc = tmp_path / "csrc"
    shutil.copytree(CSRC, csrc)
    src = (csrc / "muon_abi.hip").read_text()
    assert src.count(old) == 1, old
    (csrc / "muon_abi.hip").write_text(src.replace(old, new))
    run = _check(tmp_path, csrc)
    assert run.returncode != 0 and failure in run.stdout, run.stdout[-2000:]
