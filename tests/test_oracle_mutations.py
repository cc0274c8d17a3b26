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
    # a query-head group read against the KV head of its first head's interleaved index
    "interleaved_head_groups": ("Hkv * D, g, D, scale", "Hkv * D, (g * G) % Hkv, D, scale"),
    "diagonal_excluded": ("const int64_t n = last_key - first_key + 1;",
                          "const int64_t n = last_key - first_key;"),
    "scale_dropped": ("scores[hh * n + t] = scale * dot[hh];", "scores[hh * n + t] = dot[hh];"),
    "score_sign_flipped": ("scores[hh * n + t] = scale * dot[hh];",
                           "scores[hh * n + t] = -scale * dot[hh];"),
    "not_normalised": ("const double p = exp(scores[hh * n + t] - mx[hh]) / sum[hh];",
                       "const double p = exp(scores[hh * n + t] - mx[hh]);"),
    "lse_without_max": ("out_lse[hh * lse_stride] = mx[hh] + log(sum[hh]);",
                        "out_lse[hh * lse_stride] = log(sum[hh]);"),
    "value_rows_from_keys": ("const uint16_t* v_row = v + ", "const uint16_t* v_row = k + "),
    "query_head_of_group_leader": ("qt[d * G + hh] = bf16_bits_to_double(q_rows[hh * D + d]);",
                                   "qt[d * G + hh] = bf16_bits_to_double(q_rows[d]);"),
    "attends_across_sequences": [("scale, cu_seqlens[s], pos,", "scale, 0, pos,"),
                                 ("(size_t)(G * (longest > 0 ? longest : 1) + 3 * G + G * D + D));",
                                  "(size_t)(G * (T > 0 ? T : 1) + 3 * G + G * D + D));")],
    "no_max_shift": ("l += exp(x[t] - m);", "l += exp(x[t]);"),
    "float32_dot": ("dot[hh] += qt[d * G + hh] * kd;",
                    "dot[hh] = (float)(dot[hh] + qt[d * G + hh] * kd);"),
    "keyrange_end_inclusive": ("(key_end - 1 < pos) ? key_end - 1 : pos",
                               "(key_end < pos) ? key_end : pos"),
    "keyrange_begin_ignored": ("const int64_t first = key_begin > 0 ? key_begin : 0;",
                               "const int64_t first = 0;"),
    "keyrange_empty_lse_zero": ("lse_out[(h0 + hh) * ntok + ti] = -INFINITY;",
                                "lse_out[(h0 + hh) * ntok + ti] = 0.0;"),
    "bidirectional_masked": ("scale, 0, S - 1,", "scale, 0, pos,"),
    "bidirectional_misses_last_key": ("scale, 0, S - 1,", "scale, 0, S - 2 + (S == 1),"),
    "rope_sin_sign": ("o[i + half] = hi * c + lo * sn;", "o[i + half] = hi * c - lo * sn;"),
    "rope_frequency_exponent": ("pow(theta, -2.0 * (double)i / (double)D)",
                                "pow(theta, -1.0 * (double)i / (double)D)"),
    "rope_adjacent_pairs": ("const double lo = o[i], hi = o[i + half];",
                            "const double lo = o[i], hi = o[i ^ 1];"),
    "norm_sum_not_mean": ("sqrt(ss / (double)D + eps)", "sqrt(ss + eps)"),
    "norm_eps_outside_root": ("sqrt(ss / (double)D + eps)", "(sqrt(ss / (double)D) + eps)"),
    "norm_weight_ignored": ("o[d] = o[d] * inv * bf16_bits_to_double(weight[d]);",
                            "o[d] = o[d] * inv;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    edits = MUTANTS[name]
    if isinstance(edits, tuple):
        edits = [edits]
    with open(oracle.SOURCE) as f:
        src = f.read()
    for old, new in edits:
        assert src.count(old) >= 1, f"mutation site for {name} not found"
        src = src.replace(old, new)   # every occurrence: both entry points share the mistake
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


def _merge_plain_mean(o_parts, lse_parts):
    """Mistake: parts averaged with equal weights."""
    import numpy as np

    o = np.asarray(o_parts).mean(axis=0)
    return o, np.log(np.exp(np.asarray(lse_parts)).sum(axis=0))


_RIGHT_MERGE = oracle.merge_partials


def _merge_lse_is_max(o_parts, lse_parts):
    """Mistake: the union's LSE taken as the largest part's LSE."""
    import numpy as np

    o, _ = _RIGHT_MERGE(o_parts, lse_parts)
    return o, np.asarray(lse_parts).max(axis=0)


def _merge_not_renormalised(o_parts, lse_parts):
    """Mistake: part weights exp(lse_c - max) used without dividing by their sum."""
    import numpy as np

    lse_parts = np.asarray(lse_parts)
    m = lse_parts.max(axis=0)
    w = np.exp(lse_parts - m)
    o = (w.transpose(0, 2, 1)[..., None] * np.asarray(o_parts)).sum(axis=0)
    return o, m + np.log(w.sum(axis=0))


@pytest.mark.parametrize("wrong", [_merge_plain_mean, _merge_lse_is_max, _merge_not_renormalised],
                         ids=lambda f: f.__name__.lstrip("_"))
def test_wrong_merge_is_caught(wrong, monkeypatch):
    from oracle_pins import pin_merge_of_key_partition

    monkeypatch.setattr(oracle, "merge_partials", wrong)
    with pytest.raises(AssertionError):
        pin_merge_of_key_partition(oracle.default())


_RIGHT_POOL = oracle.pool_tokens


def _pool_divides_by_factor(x, begin, end, factor):
    """Mistake: the short last group is divided by the full factor."""
    import numpy as np

    out = _RIGHT_POOL(x, begin, end, factor)
    L = end - begin
    rem = L % factor
    if rem:
        out[begin + L // factor] *= rem / factor
    return out


def _pool_drops_tail(x, begin, end, factor):
    """Mistake: the tokens after the span are not copied (output too short)."""
    out = _RIGHT_POOL(x, begin, end, factor)
    return out[: out.shape[0] - (x.shape[0] - end)] if end < x.shape[0] else out


def _pool_first_of_group(x, begin, end, factor):
    """Mistake: subsampling (first token of each group) instead of averaging."""
    import numpy as np

    xf = _RIGHT_POOL(x, 0, 0, 1)
    out = _RIGHT_POOL(x, begin, end, factor)
    g = (end - begin + factor - 1) // factor
    out[begin:begin + g] = xf[begin:end:factor]
    return out


@pytest.mark.parametrize("wrong", [_pool_divides_by_factor, _pool_drops_tail,
                                   _pool_first_of_group], ids=lambda f: f.__name__.lstrip("_"))
def test_wrong_pooling_is_caught(wrong, monkeypatch):
    from oracle_pins import pin_pool_tokens

    monkeypatch.setattr(oracle, "pool_tokens", wrong)
    with pytest.raises(AssertionError):
        pin_pool_tokens(oracle.default())
