"""Plant plausible mistakes in a copy of the oracle and check the pins catch them.

Each mutant is oracle.c with one textual edit, compiled with gcc into a
temporary directory (the committed oracle is never touched).  The pin suite
tests/test_oracle_pins.py then runs against the mutant in a subprocess and
must fail.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "dropped_scale": ("scores[j] = scale * dot;", "scores[j] = dot;"),
    "wrong_sign": ("const double p = exp(scores[j] - m);", "const double p = exp(m - scores[j]);"),
    "gqa_index": ("const int g = h / G;", "const int g = h % Hkv;"),
    "kv_layout_transposed": ("const int64_t k_off = ((kv0 + j) * Hkv + g) * (int64_t)D;",
                             "const int64_t k_off = ((kv0 + j) + g * Hkv) * (int64_t)D;"),
    "causal_off_by_one": ("return j <= i + (n_kv - n_q);", "return j < i + (n_kv - n_q);"),
    "causal_top_left": ("return j <= i + (n_kv - n_q);", "return j <= i;"),
    "lse_log_base": ("*lse_out = m + log(l);", "*lse_out = m + log2(l);"),
    "merge_drops_l": ("const double w = li * exp(m_part[(int64_t)i * rows + r] - M);",
                      "const double w = exp(m_part[(int64_t)i * rows + r] - M);"),
    "split_range_short": ("r[1] = lo + c < n ? lo + c : n;", "r[1] = lo + c - 1 < n ? lo + c - 1 : n;"),
    "f16_exponent_bias": ("mag = ldexp((double)(f + 1024), e - 25);",
                          "mag = ldexp((double)(f + 1024), e - 24);"),
    "empty_row_lse": ("*lse_out = -INFINITY;\n    return;", "*lse_out = 0.0;\n    return;"),
    "flat_piece_end": ("const int64_t piece_end = (pos / c + 1) * c;",
                       "const int64_t piece_end = pos + c;"),
    "flat_bound_loose": ("int64_t s = (max_kv_len - 1 + c - 1) / c + 1;",
                         "int64_t s = (max_kv_len + c - 1) / c;"),
    "value_index_dropped": ("o_row[d] += p * load_elem(v, dtype, v_off + d);",
                            "o_row[d] += p * load_elem(v, dtype, v_off);"),
}


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation site for {name} not unique"
    mutant_c = tmp_path / "oracle_mutant.c"
    mutant_c.write_text(source.replace(old, new))
    so = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-o", str(so),
                    str(mutant_c), "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIBRARY_VARIANT=str(so), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"
    assert "failed" in r.stdout or "error" in r.stdout.lower()
