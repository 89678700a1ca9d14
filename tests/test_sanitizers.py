"""CPU builds of the C oracle and of the library's host-side validation under
AddressSanitizer and UndefinedBehaviorSanitizer (host code only: the device code is built
without them).  Each driver under tests/sanitize/ runs its code paths, edge cases
included, and any sanitizer report fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r.stdout


def test_oracle_under_asan_ubsan(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_driver")
    run(["gcc", "-O1", "-g", "-fopenmp", *SAN, os.path.join(ROOT, "oracle", "oracle.c"),
         os.path.join(HERE, "oracle_driver.c"), "-o", exe, "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", OMP_NUM_THREADS="2")
    assert "all checks passed" in run([exe], env=env)


def test_host_validation_under_asan_ubsan(tmp_path):
    if not (os.path.exists(HIPCC) and shutil.which("g++")):
        pytest.skip("hipcc or g++ not found")
    obj, drv, exe = (str(tmp_path / n) for n in ("flashfwd.o", "driver.o", "host_driver"))
    # the device code is compiled without sanitizers (-fno-gpu-sanitize); the host pass
    # of flashfwd.hip carries them
    run([HIPCC, "-c", "-x", "hip", "--offload-arch=gfx950", "-fno-gpu-sanitize", *SAN, "-O1",
         "-g", "-std=c++17", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"),
         "-I", os.path.join(ROOT, "io_aware_attention_amd", "csrc"),
         os.path.join(ROOT, "io_aware_attention_amd", "csrc", "flashfwd.hip"), "-o", obj])
    run(["g++", "-c", "-O1", "-g", *SAN, "-I", os.path.join(ROOT, "include"),
         os.path.join(HERE, "host_driver.cpp"), "-o", drv])
    run([HIPCC, "-fno-gpu-sanitize", *SAN, obj, drv, "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    assert "all checks passed" in run([exe], env=env)
