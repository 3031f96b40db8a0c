"""Plants plausible mistakes in a copy of the oracle and checks the pins fail.

Each mutant is oracle.c with one textual change (a dropped key/value segment,
a wrong predecessor index, a missing scale, V read from K, heads mixed, ...),
compiled on the CPU into a temporary library.  The pin suite
(test_oracle_pins.py) is run against it in a subprocess and must fail.  This
shows the pins constrain every part of the definition, not just that the
unmodified oracle agrees with itself.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "own_rows_dropped": ("return c >= 1 ? 2 * chunk_len : chunk_len;", "return chunk_len;"),
    "predecessor_is_self": ("*k_off = ((c - 1) * L + j) * H * D;", "*k_off = (c * L + j) * H * D;"),
    "predecessor_row_shift": ("*k_off = ((c - 1) * L + j) * H * D;",
                              "*k_off = ((c - 1) * L + (j + 1) % L) * H * D;"),
    "scale_dropped": ("s[j] = scale * acc;", "s[j] = acc;"),
    "v_read_from_k": ("out[d] += w * load_elem(vb, dtype, vo + d);",
                      "out[d] += w * load_elem(kb, dtype, ko + d);"),
    "heads_mixed": ("k_off += src->h * src->D;", "k_off += 0;"),
    "cache_v_from_k_slot": ("*v_off = ((c * 2 + 1) * L + j) * H * D;",
                            "*v_off = ((c * 2 + 0) * L + j) * H * D;"),
    "softmax_sign": ("s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    "not_normalised": ("double w = s[j] / z;", "double w = s[j];"),
    "cache_ignored": ("*from_cache = 1;", "*from_cache = 0; *k_off = ((c - 1) * L + j) * H * D; *v_off = *k_off;"),
    "dot_truncated": ("for (int64_t d = 0; d < D; ++d)\n            acc +=",
                      "for (int64_t d = 0; d + 1 < D; ++d)\n            acc +="),
    # window step
    "window_next_chunk_is_self": ("chunk[j] = c + 1;", "chunk[j] = c;"),
    "window_query_row_shift": ("const int64_t q_row = r < L ? r : r - L;",
                               "const int64_t q_row = r < L ? r : (r - L + 1) % L;"),
    "window_cache_slot_off_by_one": ("*ko = (((c * 2 + 0) * L + row) * H + h) * D;",
                                     "*ko = ((((c - 1) * 2 + 0) * L + row) * H + h) * D;"),
    "window_heads_mixed": ("*ko = ((chunk * L + row) * H + h) * D;",
                           "*ko = ((chunk * L + row) * H + 0) * D;"),
    "ring_wrap_clamped": ("return p < 0 ? p + slots : p;", "return p < 0 ? 0 : p;"),
    "ring_predecessor_older": ("slot[nk] = oracle_ring_slot(slots, tail_slot, c - 1);",
                               "slot[nk] = oracle_ring_slot(slots, tail_slot, c + 1);"),
    "window_predecessor_dropped": ("if (c >= 1)\n        for (int64_t r = 0; r < chunk_len; ++r, ++j) {",
                                   "if (0)\n        for (int64_t r = 0; r < chunk_len; ++r, ++j) {"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(before) == 1, f"mutation anchor for {name} not found exactly once"
    mutant = tmp_path / "oracle_mutant.c"
    mutant.write_text(src.replace(before, after))
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", str(mutant),
                    "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, CHUNKATTN_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch mutant {name}:\n{r.stdout[-2000:]}"
    assert "failed" in r.stdout
