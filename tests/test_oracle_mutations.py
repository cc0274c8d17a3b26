"""Each plausible mistake planted in a copy of the oracle trips a pin.

The copies are compiled from ``oracle/oracle.c`` with one text substitution
each, in a temporary folder, on the CPU.  A mutant that passed every pin would
show that the pins cannot tell that mistake from the definition.
"""

import os

import pytest

import oracle
from oracle_pins import ALL_PINS

MUTANTS = {
    "interleaved_head_groups": ("const int64_t g = h / G;", "const int64_t g = h % Hkv;"),
    "diagonal_excluded": ("const int64_t n = last_key - first_key + 1;",
                          "const int64_t n = last_key - first_key;"),
    "scale_dropped": ("scores[t] = scale * dot;", "scores[t] = dot;"),
    "score_sign_flipped": ("scores[t] = scale * dot;", "scores[t] = -scale * dot;"),
    "not_normalised": ("const double p = exp(scores[t] - m) / l;",
                       "const double p = exp(scores[t] - m);"),
    "lse_without_max": ("return m + log(l);", "return log(l);"),
    "value_rows_from_keys": ("const uint16_t* v_row = v + ", "const uint16_t* v_row = k + "),
    "query_head_of_group_leader": ("q + (pos * Hq + h) * D", "q + (pos * Hq + g * G) * D"),
    "attends_across_sequences": [("cu_seqlens[s], pos, scores", "0, pos, scores"),
                                 ("double* scores = (double*)malloc(sizeof(double) * (size_t)(longest > 0 ? longest : 1));",
                                  "double* scores = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));")],
    "no_max_shift": ("l += exp(scores[t] - m);", "l += exp(scores[t]);"),
    "float32_dot": ("double dot = 0.0;", "float dot = 0.0f;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    edits = MUTANTS[name]
    if isinstance(edits, tuple):
        edits = [edits]
    with open(oracle.SOURCE) as f:
        src = f.read()
    for old, new in edits:
        assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
        src = src.replace(old, new)
    mutant_src = tmp_path / "oracle_mutant.c"
    mutant_src.write_text(src)
    lib = oracle.build(str(mutant_src), str(tmp_path / "liboracle_mutant.so"))
    orc = oracle.Oracle(os.fspath(lib))
    failed = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"no pin notices the mutant {name}"
