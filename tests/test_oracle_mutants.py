"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of oracle.c (on the CPU, in a
temporary directory), rebuilds it and runs the pin suite against it; the
suite has to fail.  The planted mistakes are the kinds the pins are meant to
catch: a dropped term, a flipped sign, a wrong index or transposed operand,
a reversed tie-break, a missing normalisation, a mis-scaled or mis-gated
shared expert, and a wrong slot index in the routing plan.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "dropped_last_term": ("for (int c = 0; c < n; ++c) s +=",
                          "for (int c = 0; c < n - 1; ++c) s +="),
    "silu_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "up_rows_are_gate_rows": ("W13, (size_t)(I + i) * d, dt, d);",
                              "W13, (size_t)(i) * d, dt, d);"),
    "down_transposed": ("elem(W2, dt, (size_t)r * I + i)", "elem(W2, dt, (size_t)i * d + r)"),
    "tie_prefers_higher_index": ("if (best < 0 || v > bv)", "if (best < 0 || v >= bv)"),
    "bias_subtracted": ("if (bias) l += (double)bias", "if (bias) l -= (double)bias"),
    "weights_not_normalised": ("w[j] = exp((double)(float)logits[ids[j]] - m) / z;",
                               "w[j] = exp((double)(float)logits[ids[j]] - m);"),
    "shared_half_weight": ("for (int r = 0; r < d; ++r) o[r] += y[r];",
                           "for (int r = 0; r < d; ++r) o[r] += 0.5 * y[r];"),
    "combine_shared_inverted": ("if (has_shared) s +=", "if (!has_shared) s +="),
    "plan_token_not_slot": ("slots[pos++] = s;", "slots[pos++] = s / k;"),
    "latent_rows_transposed": ("latent[(size_t)t * L + j] = dot(X, (size_t)t * d, Wl, (size_t)j * d, dt, d);",
                               "latent[(size_t)t * L + j] = dot(X, (size_t)t * d, Wl, (size_t)j, dt, d);"),
    "residual_transposed": ("elem(R, dt, (size_t)b * N + n)", "elem(R, dt, (size_t)n * B + b)"),
    "residual_dropped": ("dot(X, (size_t)b * K, W, (size_t)n * K, dt, K) +\n          elem(R",
                         "dot(X, (size_t)b * K, W, (size_t)n * K, dt, K) +\n          0.0 * elem(R"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    assert src.count(old) >= 1, "mutation anchor not found: %s" % old
    (tmp_path / "oracle").mkdir()
    (tmp_path / "oracle" / "oracle.c").write_text(src.replace(old, new))
    for f in ("oracle.py", "__init__.py"):
        shutil.copy(os.path.join(ROOT, "oracle", f), tmp_path / "oracle" / f)
    shutil.copytree(os.path.join(ROOT, "moe_block_skinny_amd"), tmp_path / "moe_block_skinny_amd",
                    ignore=shutil.ignore_patterns("*.so", "csrc", "__pycache__"))
    (tmp_path / "tests").mkdir()
    for f in ("conftest.py", "test_oracle_pins.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), tmp_path / "tests" / f)
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), tmp_path / "tests" / "golden")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py"], cwd=tmp_path, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0, "pins did not catch mutant %s:\n%s" % (name, r.stdout[-2000:])
    assert "failed" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]
