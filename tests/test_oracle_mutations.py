"""The oracle pins catch plausible mistakes.

Each case plants one mistake in a temporary copy of the oracle's C source
(never in the real one), builds it, and runs the pin suite against it through
LOOM_ORACLE_LIB; the suite must fail.  The mistakes are the ones a careless
transcription of the pages would make: an off-by-one tile condition, a dropped
lane or tail row, a corrupted row, unsigned bytes, a transposed weight index,
the wrong scale, an ignored row stride.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = {
    "tile loop stops one tile early": ("while (remaining >= tile) {", "while (remaining > tile) {"),
    "row reduction drops the last lane": ("row_sum = row_sum + values[source_row * lanes + l];",
                                          "row_sum = row_sum + values[source_row * lanes + l] * (l < 31);"),
    "row sums drop the last tail row": ("for (int64_t t = 0; t < tail_count; ++t) {",
                                        "for (int64_t t = 0; t < tail_count - 1; ++t) {"),
    "segment walk corrupts a row": ("float v = x[(begin + r) * cols + c];",
                                    "float v = x[(begin + r) * cols + c] + (r == 9 ? 1.0f : 0.0f);"),
    "bytes read as unsigned": ("(int64_t)w[r * k + i] * (int64_t)x[b * k + i]",
                               "(int64_t)(uint8_t)w[r * k + i] * (int64_t)x[b * k + i]"),
    "weights transposed": ("(int64_t)w[r * k + i] * (int64_t)x[b * k + i]",
                           "(int64_t)w[i * rows + r] * (int64_t)x[b * k + i]"),
    "vector scale index fixed": ("if (x_scale) y = y * x_scale[b];", "if (x_scale) y = y * x_scale[0];"),
    "row stride ignored": ("row_sum_one(x + r * row_stride, cols", "row_sum_one(x + r * cols, cols"),
    "packed-dot bytes unsigned": ("int8_t byte = (int8_t)(uint8_t)(word >> (8 * j));",
                                  "int byte = (uint8_t)(word >> (8 * j));"),
    "packed-dot stream by division": ("int64_t stream = o % streams;", "int64_t stream = (o / streams) % streams;"),
    "packed-dot scale ignored": ("float v = (float)byte * scale;", "float v = (float)byte;"),
    "guarded rows: inner loop one short": ("for (int64_t column = 0; column < columns; ++column) {",
                                           "for (int64_t column = 0; column + 1 < columns; ++column) {"),
    "guarded rows: lane guard ignored": ("if (active) value = values[", "value = values["),
    "guarded rows: row guard off by one": ("if (row < count) {", "if (row <= count && row < 63) {"),
    "routed combine: signed id check": ("if ((uint64_t)id >= (uint64_t)num_rows) continue;",
                                        "if ((int32_t)id >= num_rows) continue; if ((int32_t)id < 0) id = 0;"),
    "routed combine: last row treated as missing": ("if ((uint64_t)id >= (uint64_t)num_rows) continue;",
                                                    "if ((uint64_t)id + 1 >= (uint64_t)num_rows) continue;"),
    "routed combine: weight of the wrong route": ("float w = weights[t * routes + i];",
                                                 "float w = weights[t * routes + (i + 1) % routes];"),
    "packed-dot byte order reversed": ("int8_t byte = (int8_t)(uint8_t)(word >> (8 * j));",
                                       "int8_t byte = (int8_t)(uint8_t)(word >> (8 * (3 - j)));"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(os.path.join(ROOT, "oracle", "loom_oracle.c")).read()
    assert old in src, f"mutation target not found: {old}"
    mutated = tmp_path / "loom_oracle_mutant.c"
    mutated.write_text(src.replace(old, new, 1))
    so = tmp_path / "libloom_oracle_mutant.so"
    subprocess.run(["gcc", *oracle.CFLAGS, "-o", str(so), str(mutated), "-lm"], check=True)
    env = dict(os.environ, LOOM_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins passed with a planted mistake ({name}):\n{r.stdout[-2000:]}"


def test_unmutated_oracle_passes_pins(tmp_path):
    so = tmp_path / "libloom_oracle_copy.so"
    subprocess.run(["gcc", *oracle.CFLAGS, "-o", str(so), os.path.join(ROOT, "oracle", "loom_oracle.c"), "-lm"],
                   check=True)
    env = dict(os.environ, LOOM_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:]
