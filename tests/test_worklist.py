"""Host-side unit test of the tiled kernels' work lists (worklist.h): the workgroup -> item
map is a permutation of every list, idle exactly past the unit count, keeps each XCD on its
own unit slots, runs each XCD's items heaviest first in (rank, unit, sub) order, and in
snake mode mirrors every other round of resident workgroups.  No GPU: the index functions
are compiled for the host."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def test_work_lists_are_ordered_permutations(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    exe = str(tmp_path / "worklist_check")
    r = subprocess.run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O2", "-std=c++17",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        "-I", os.path.join(ROOT, "io_aware_attention_amd", "csrc"),
                        os.path.join(ROOT, "tests", "native", "worklist_check.cpp"),
                        "-o", exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "all checks passed" in r.stdout, r.stdout[-3000:] + r.stderr[-2000:]
