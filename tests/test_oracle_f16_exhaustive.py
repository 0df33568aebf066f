"""The C++ oracle's own fp32 -> fp16 round-to-nearest-even conversion (used for every group
step) equals the host's F16C instruction on all 2^32 fp32 bit patterns (CPU only)."""
import os
import subprocess

import pytest

from oracle import cpp_oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _has_f16c():
    try:
        return "f16c" in open("/proc/cpuinfo").read().split()
    except OSError:
        return False


@pytest.mark.skipif(not _has_f16c(), reason="host CPU has no F16C instruction to compare with")
def test_fp32_to_fp16_all_patterns_match_f16c(tmp_path):
    exe = tmp_path / "f16_exhaustive"
    r = subprocess.run(["g++", "-O2", "-mf16c", "-fopenmp", os.path.join(HERE, "native", "f16_exhaustive.cpp"),
                        "-o", str(exe), "-ldl"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe), cpp_oracle.LIB_PATH], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and "mismatches 0" in r.stdout, r.stdout + r.stderr
