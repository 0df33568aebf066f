"""The oracle's pins are sharp: each planted mistake in a private copy of the oracle
makes the pin suite fail.  The copy lives in a temporary directory; the real oracle
is never modified."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = {
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


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(os.path.join(ROOT, "oracle", "awq_oracle.py")).read()
    assert old in src, f"mutation {name} no longer applies"
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle",
                    ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copytree(os.path.join(ROOT, "gen"), tmp_path / "gen", ignore=shutil.ignore_patterns("__pycache__"))
    (tmp_path / "tests").mkdir()
    for f in ("conftest.py", "test_oracle_pins.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), tmp_path / "tests" / f)
    (tmp_path / "oracle" / "awq_oracle.py").write_text(src.replace(old, new, 1))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "tests"],
                       cwd=tmp_path, capture_output=True, text=True, timeout=300)
    assert r.returncode == 1, f"planted mistake {name} was not caught:\n{r.stdout[-2000:]}"
