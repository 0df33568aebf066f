"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Two builds in a temporary copy of the tree, each running existing CPU tests unchanged:
- the C++ oracle, compiled by g++ with ASan+UBSan, under the oracle pins and the
  C++/numpy cross-check;
- libawq's host code (argument checks, workspace sizing, the C-ABI entry points up to
  the first GPU call), compiled by hipcc with the sanitizers on the host pass only, under
  the ABI tests.  The device code is built as usual; no test here touches a GPU.
A sanitizer report aborts the process, so any finding fails the test."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GCC_ASAN = "/usr/lib/gcc/x86_64-linux-gnu/11/libasan.so"
CLANG_ASAN = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))

ORACLE_SAN_FLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                    "-fno-sanitize-recover=undefined", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                    "-std=c++17"]
HOST_SAN_FLAGS = ["-Xarch_host", "-fsanitize=address",
                  "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer"]


def _env(preload):
    env = dict(os.environ)
    env["LD_PRELOAD"] = preload
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


def _copy_tests(tmp_path, files):
    (tmp_path / "tests").mkdir()
    for f in ("conftest.py", "layout.py", *files):
        shutil.copy(os.path.join(ROOT, "tests", f), tmp_path / "tests" / f)
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), tmp_path / "tests" / "golden")


def _pytest(tmp_path, files, env):
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *files],
                          cwd=tmp_path, capture_output=True, text=True, timeout=900, env=env)


@pytest.mark.slow
@pytest.mark.skipif(not os.path.exists(GCC_ASAN), reason="gcc's libasan is not installed")
def test_oracle_under_asan_ubsan(tmp_path):
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle",
                    ignore=shutil.ignore_patterns("__pycache__", "*.so", "*.tmp"))
    shutil.copytree(os.path.join(ROOT, "gen"), tmp_path / "gen", ignore=shutil.ignore_patterns("__pycache__"))
    files = ["test_oracle_pins.py", "test_oracle_cross.py"]
    _copy_tests(tmp_path, files)
    src = tmp_path / "oracle" / "awq_oracle.cpp"
    r = subprocess.run(["g++", *ORACLE_SAN_FLAGS, str(src), "-o", str(tmp_path / "oracle" / "liboracle.so")],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    r = _pytest(tmp_path, [f"tests/{f}" for f in files], _env(GCC_ASAN))
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])


@pytest.mark.slow
@pytest.mark.skipif(not CLANG_ASAN, reason="clang's ASan runtime is not installed")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    for d in ("weight_only_quantization_gemm_amd", "include", "gen", "oracle"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("__pycache__", "_build", "*.so", "*.tmp"))
    _copy_tests(tmp_path, ["test_abi.py"])
    script = ("import sys; sys.path.insert(0, '.');"
              "from weight_only_quantization_gemm_amd import build as b;"
              f"b.FLAGS = b.FLAGS + {HOST_SAN_FLAGS!r};"
              "b.build()")
    r = subprocess.run([sys.executable, "-c", script], cwd=tmp_path, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stderr[-3000:]
    nm = subprocess.run(["nm", "-D", str(tmp_path / "weight_only_quantization_gemm_amd" / "libawq.so")],
                        capture_output=True, text=True)
    assert "__asan_" in nm.stdout, "the host pass was not instrumented"
    r = _pytest(tmp_path, ["tests/test_abi.py"], _env(CLANG_ASAN[-1]))
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
