"""The oracle's pins are sharp: each planted mistake in a private copy of the oracle makes
the pin suite fail.  The copy lives in a temporary directory; the real oracle is never
modified.  Mistakes are planted both in the C++ oracle (awq_oracle.cpp, rebuilt in the copy
and checked by tests/test_oracle_pins.py and the exhaustive fp16 check) and in the numpy
implementation (awq_oracle.py, checked by tests/test_oracle_pins_numpy.py)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS_NUMPY = {
    "step_over_16": ("(hi - lo) / qmax", "(hi - lo) / np.float32(16)"),
    "floor_not_rint": ("np.rint(Vg / sc[:, :, None])", "np.floor(Vg / sc[:, :, None])"),
    "round_after_zero": ("np.rint(Vg / sc[:, :, None]) + z[:, :, None]",
                         "np.rint(Vg / sc[:, :, None] + z[:, :, None])"),
    "unrounded_scale": ("sc = sc16.astype(np.float32)", "sc = step"),
    "signed_mean": ("(np.abs(X[r0:r0 + 4096]).astype(np.float64)", "(X[r0:r0 + 4096].astype(np.float64).clip(0)"),
    "multiply_by_s": ("dequantize(q, z, sc16, group) / np.asarray(s", "dequantize(q, z, sc16, group) * np.asarray(s"),
    "range_without_zero": ("lo = np.minimum(Vg.min(axis=2), np.float32(0.0))", "lo = Vg.min(axis=2)"),
    "zero_point_sign": ("z = np.clip(np.rint(-lo / sc)", "z = np.clip(np.rint(lo / sc)"),
    "tie_to_last": ("if losses[i] < losses[best]:", "if losses[i] <= losses[best]:"),
    "loss_per_row_only": ("/ (np.float64(M) * np.float64(N)))\n\n\ndef gram", "/ (np.float64(M)))\n\n\ndef gram"),
    "gram_perturbed": ("return X.T @ X", "return X.T @ X * 1.0000001"),
    "levels_not_minus_one": ("qmax = np.float32(2 ** bits - 1)", "qmax = np.float32(2 ** bits)"),
    "fixed_four_bit_range": ("qmax = np.float32(2 ** bits - 1)", "qmax = np.float32(15)"),
    "kept_columns_not_restored": ("    E[:, np.asarray(keep, dtype=np.int64)] = 0.0\n", "\n"),
    "smallest_channels_kept": ("key=lambda k: (-v[k], k)", "key=lambda k: (v[k], k)"),
    "scaled_input_multiplies": ("return (x32 / np.asarray(s, dtype=np.float32)[None, :])",
                                "return (x32 * np.asarray(s, dtype=np.float32)[None, :])"),
    "scaled_input_in_fp16": ("return (x32 / np.asarray(s, dtype=np.float32)[None, :]).astype(np.float16)",
                             "return (x32.astype(np.float16) / np.asarray(s, dtype=np.float16)[None, :])"),
    "gemm_wrong_group": ("zz = np.repeat(np.asarray(z, dtype=np.float64), group, axis=1)",
                         "zz = np.tile(np.asarray(z, dtype=np.float64), (1, group))"),
}

MUTATIONS_CPP = {
    "step_over_16": ("g.step = range / qmax;", "g.step = range / (qmax + 1.0f);"),
    "floor_not_rint": ("std::nearbyint(v[i] / g.sc) + g.z", "std::floor(v[i] / g.sc) + g.z"),
    "round_after_zero": ("std::nearbyint(v[i] / g.sc) + g.z", "std::nearbyint(v[i] / g.sc + g.z)"),
    "unrounded_scale": ("g.sc = f16_to_f32(g.sc16);", "g.sc = g.step;"),
    "signed_mean": ("s += abs_units(X[t * K + k]);", "s += (X[t * K + k] >> 15) ? 0 : abs_units(X[t * K + k]);"),
    "multiply_by_s": ("E[n * K + k] = wh / sd - ", "E[n * K + k] = wh * sd - "),
    "range_without_zero": ("g.lo = 0.0f;\n  g.hi = 0.0f;", "g.lo = v[0];\n  g.hi = v[0];"),
    "zero_point_sign": ("std::nearbyint(-g.lo / g.sc)", "std::nearbyint(g.lo / g.sc)"),
    "tie_to_last": ("if (losses[i] < losses[b]) b = i;", "if (losses[i] <= losses[b]) b = i;"),
    "loss_per_row_only": ("  return total / ((double)M * (double)N);\n}\n\n// G = X^T X",
                          "  return total / (double)M;\n}\n\n// G = X^T X"),
    "gram_perturbed": ("g[j] += xi * (double)xr[j];", "g[j] += xi * (double)xr[j] * 1.0000001;"),
    "levels_not_minus_one": ("const float qmax = (float)((1 << bits) - 1);", "const float qmax = (float)(1 << bits);"),
    "fixed_four_bit_range": ("const float qmax = (float)((1 << bits) - 1);", "const float qmax = 15.0f;"),
    "kept_columns_not_restored": ("for (int64_t n = 0; n < N; ++n) E[n * K + k] = 0.0;", "(void)k;"),
    "smallest_channels_kept": ("return v[i] > v[j];", "return v[i] < v[j];"),
    "scaled_input_multiplies": ("f16_to_f32(x[m * K + k]) / s[k]", "f16_to_f32(x[m * K + k]) * s[k]"),
    "scaled_input_in_fp16": ("f16_to_f32(x[m * K + k]) / s[k]",
                             "f16_to_f32(f32_to_f16(f16_to_f32(x[m * K + k]) / f16_to_f32(f32_to_f16(s[k]))))"),
    "gemm_wrong_group": ("wrow[k] = dequant(q[n * K + k], z[n * G + k / group], sc16[n * G + k / group]);",
                         "wrow[k] = dequant(q[n * K + k], z[n * G + k % G], sc16[n * G + k / group]);"),
    "fp16_ties_away": ("(rem == half && (kept & 1u))", "(rem == half)"),
    "fp16_no_subnormals": ("const int shift = e >= -14 ? 13 : -1 - e;", "const int shift = e >= -14 ? 13 : 99;"),
}


def _copy_tree(tmp_path):
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle",
                    ignore=shutil.ignore_patterns("__pycache__", "*.so", "*.tmp"))
    shutil.copytree(os.path.join(ROOT, "gen"), tmp_path / "gen", ignore=shutil.ignore_patterns("__pycache__"))
    (tmp_path / "tests").mkdir()
    for f in ("conftest.py", "test_oracle_pins.py", "test_oracle_pins_numpy.py", "test_oracle_f16_exhaustive.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), tmp_path / "tests" / f)
    shutil.copytree(os.path.join(ROOT, "tests", "native"), tmp_path / "tests" / "native")


def _run_pins(tmp_path, files):
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *files],
                          cwd=tmp_path, capture_output=True, text=True, timeout=600)


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTATIONS_NUMPY))
def test_pins_catch_planted_mistake_numpy(name, tmp_path):
    old, new = MUTATIONS_NUMPY[name]
    src = open(os.path.join(ROOT, "oracle", "awq_oracle.py")).read()
    assert old in src, f"mutation {name} no longer applies"
    _copy_tree(tmp_path)
    (tmp_path / "oracle" / "awq_oracle.py").write_text(src.replace(old, new, 1))
    shutil.copy(os.path.join(ROOT, "oracle", "liboracle.so"), tmp_path / "oracle" / "liboracle.so")
    r = _run_pins(tmp_path, ["tests/test_oracle_pins_numpy.py"])
    assert r.returncode == 1, f"planted mistake {name} was not caught:\n{r.stdout[-2000:]}"


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTATIONS_CPP))
def test_pins_catch_planted_mistake_cpp(name, tmp_path):
    old, new = MUTATIONS_CPP[name]
    src = open(os.path.join(ROOT, "oracle", "awq_oracle.cpp")).read()
    assert src.count(old) == 1, f"mutation {name} no longer applies once"
    _copy_tree(tmp_path)
    (tmp_path / "oracle" / "awq_oracle.cpp").write_text(src.replace(old, new, 1))
    r = subprocess.run([sys.executable, "-c", "from oracle import cpp_oracle; cpp_oracle.build()"], cwd=tmp_path,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    r = _run_pins(tmp_path, ["tests/test_oracle_pins.py", "tests/test_oracle_f16_exhaustive.py"])
    assert r.returncode == 1, f"planted mistake {name} was not caught:\n{r.stdout[-2000:]}"
