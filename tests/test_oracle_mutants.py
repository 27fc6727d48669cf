"""Each planted mistake in a copy of the oracle must fail at least one pin.

The copies are built from ``oracle/attn_oracle.c`` with one textual change
each, on the CPU, into a temporary directory. Every change keeps all memory
accesses inside the input arrays.
"""
import os

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.library_path()), "attn_oracle.c")

MUTANTS = {
    "dropped_scale": [("s[j] = scale * dot;", "s[j] = dot;")],
    "exp_sign": [("s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);")],
    "no_max_subtraction": [("s[j] = exp(s[j] - m);", "s[j] = exp(s[j]);"),
                           ("*lse = m + log(l);", "*lse = log(l);")],
    "lse_base2": [("*lse = m + log(l);", "*lse = m + log2(l);")],
    "lse_without_max": [("*lse = m + log(l);", "*lse = log(l);")],
    "causal_excludes_diagonal": [("causal ? i + 1 : N", "causal ? (i > 0 ? i : 1) : N")],
    "causal_one_key_too_many": [("causal ? i + 1 : N", "causal ? (i + 2 < N ? i + 2 : N) : N")],
    "causal_upper_triangle": [("const int64_t n_keys = causal ? i + 1 : N;",
                               "const int64_t n_keys = causal ? N - i : N;")],
    "transposed_k": [("dot += qi[c] * kj[c];", "dot += qi[c] * k[(c % N) * d + (j % d)];")],
    "transposed_v": [("o_row[c] += w * vj[c];", "o_row[c] += w * v[(c % N) * d + (j % d)];")],
    "wrong_head_offset": [("(size_t)bh * (size_t)N * (size_t)d", "(size_t)bh * (size_t)N")],
    "no_normalisation": [("const double w = s[j] / l;", "const double w = s[j];")],
    "output_not_cleared": [("o_row[c] = 0.0;", "o_row[c] = 1e-3;")],
    "max_is_min": [("if (s[j] > m) m = s[j];", "if (s[j] < m || j == 0) m = s[j];")],
    "last_key_dropped_from_output": [("for (int64_t j = 0; j < n_keys; ++j) {\n    const double w",
                                      "for (int64_t j = 0; j + 1 < n_keys; ++j) {\n    const double w")],
    "last_key_dropped_from_sum": [("    l += s[j];", "    l += (j + 1 < n_keys) ? s[j] : 0.0;")],
    "query_head_uses_key_length": [("const size_t qhead = (size_t)bh * (size_t)Nq * (size_t)d;",
                                    "const size_t qhead = (size_t)bh * (size_t)N * (size_t)d;")],
    "keys_counted_with_query_length": [("  const int64_t N = Nk;\n", "  const int64_t N = Nk < Nq ? Nk : Nq;\n")],
    "query_row_off_by_one": [("const double *qi = q + i * d;",
                              "const double *qi = q + ((i + 1) % N) * d;")],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    src = open(SRC).read()
    for old, new in MUTANTS[name]:
        assert old in src, "mutation anchor missing: %r" % old
        src = src.replace(old, new, 1)
    path = tmp_path / ("mutant_%s.c" % name)
    path.write_text(src)
    lib = oracle.open_oracle_library(oracle.compile_oracle(str(path), str(tmp_path / "m.so")))

    def attn(q, k, v, causal, scale, rows=None):
        return oracle.attn_oracle(q, k, v, causal=causal, scale=scale, rows=rows, lib=lib)

    failed = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            if check is oracle_pins.check_variants_agree:
                check(attn, seeds=range(10))
            else:
                check(attn)
        except AssertionError:
            failed.append(check.__name__)
            break
    assert failed, "planted mistake %r passed every pin" % name
