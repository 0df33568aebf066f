"""The Gram's work plan (which block adds up which tile over which calibration rows, and
where split tiles leave their partial sums), checked on the host: the plan's own functions
from csrc/gram.hip are compiled into tests/gram_plan_check.cpp and walked block by block."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

# K in 128-channel tiles from one tile to the 70B down projection; Mp from one 64-row
# stage (fewer rows than a flush chunk) to 131,072 calibration rows
KS = [128, 256, 384, 512, 1024, 1536, 2048, 4096, 5120, 8192, 11008, 13824, 14336, 28672]
MPS = [64, 128, 192, 256, 320, 512, 640, 1024, 4096, 8192, 65536, 131072]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc is not installed")
def test_gram_plan_covers_every_tile_once(tmp_path):
    exe = tmp_path / "gram_plan_check"
    r = subprocess.run([HIPCC, "-std=c++17", "-O1", "--offload-arch=gfx950", "-x", "hip",
                        "-I", os.path.join(ROOT, "weight_only_quantization_gemm_amd", "csrc"),
                        os.path.join(ROOT, "tests", "gram_plan_check.cpp"), "-o", str(exe)],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    cases = [f"{K}:{Mp}" for K in KS for Mp in MPS]
    r = subprocess.run([str(exe), *cases], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout[-2000:]
    lines = r.stdout.strip().splitlines()
    assert len(lines) == len(cases)
    # K = 4096 at 65,536 rows: XCD 0 runs 64 whole tiles, then 4 tiles cut 16 ways (128 blocks);
    # K = 11008: an XCD with 30 tiles in its last round sets the time, so nothing is cut
    assert "K=4096 Mp=65536 blocks=1024 split=34 " in r.stdout
    assert "K=11008 Mp=65536 blocks=3824 split=0 " in r.stdout
