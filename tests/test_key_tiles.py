"""Host-side unit test of the prefill kernel's key-tile range (tiles.h): which key tiles a
query tile visits and which of them run masked, checked against an element-by-element
visibility scan and against per-row visible intervals (windows and positions past 2^31
included).  No GPU: the range function is compiled for the host."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def test_key_tile_range_matches_visibility(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    exe = str(tmp_path / "key_tiles_check")
    r = subprocess.run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O2", "-std=c++17",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        "-I", os.path.join(ROOT, "io_aware_attention_amd", "csrc"),
                        os.path.join(ROOT, "tests", "native", "key_tiles_check.cpp"),
                        "-o", exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "all checks passed" in r.stdout, r.stdout[-3000:] + r.stderr[-2000:]
