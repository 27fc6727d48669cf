"""Each planted mistake in a copy of the backward oracle must fail at least
one pin.

The copies are built from ``oracle/attn_bwd_oracle.c`` with one textual change
each, on the CPU, into a temporary directory. Every change keeps all memory
accesses inside the input arrays. The first two are the failure signatures
that "4.4 Writing GPU Kernels with Triton" names in its Kernel 5 correctness
notes: dS without the D_i subtraction, and a dropped or doubled scale.
"""
import os

import pytest

import oracle
import oracle_bwd_pins

SRC = os.path.join(os.path.dirname(oracle.bwd_library_path()), "attn_bwd_oracle.c")

MUTANTS = {
    "dq_without_D": [("const double ds = p * (dp - D);", "const double ds = p * dp;")],
    "dkdv_without_D": [("const double ds = p * (dp - D[i]);", "const double ds = p * dp;")],
    "dq_scale_dropped": [("for (int64_t c = 0; c < d; ++c) dq[c] *= scale;", "")],
    "dq_scale_twice": [("dq[c] *= scale;", "dq[c] *= scale * scale;")],
    "dk_scale_dropped": [("for (int64_t c = 0; c < d; ++c) dk[c] *= scale;", "")],
    "ds_sign": [("const double ds = p * (dp - D);", "const double ds = p * (D - dp);"),
                ("const double ds = p * (dp - D[i]);", "const double ds = p * (D[i] - dp);")],
    "dv_from_ds": [("dv[c] += p * dout[i * d + c];", "dv[c] += ds * dout[i * d + c];")],
    "dk_from_k": [("dk[c] += ds * q[i * d + c];", "dk[c] += ds * k[i * d + c];")],
    "dq_from_v": [("dq[c] += ds * k[j * d + c];", "dq[c] += ds * v[j * d + c];")],
    "D_from_v": [("*D_out = dot(dout + i * d, o_row, d);", "*D_out = dot(dout + i * d, v + i * d, d);")],
    "dkdv_causal_row_too_many": [("const int64_t i0 = causal ? j : 0;",
                                  "const int64_t i0 = causal ? (j > 0 ? j - 1 : 0) : 0;")],
    "dkdv_causal_diagonal_dropped": [("const int64_t i0 = causal ? j : 0;",
                                      "const int64_t i0 = causal ? j + 1 : 0;")],
    "dq_dp_transposed": [("const double dp = dot(dout + i * d, v + j * d, d);\n    const double ds = p * (dp - D);",
                          "const double dp = dot(dout + j * d, v + i * d, d);\n    const double ds = p * (dp - D);")],
    "dkdv_dp_transposed": [("const double dp = dot(dout + i * d, v + j * d, d);\n    const double ds = p * (dp - D[i]);",
                            "const double dp = dot(dout + j * d, v + i * d, d);\n    const double ds = p * (dp - D[i]);")],
    "dq_unnormalised": [("const double p = exp(scale * dot(q + i * d, k + j * d, d) - m) / l;",
                         "const double p = exp(scale * dot(q + i * d, k + j * d, d) - m);")],
    "dkdv_stats_of_wrong_row": [("- m[i]) / l[i];", "- m[j]) / l[j];")],
    "dkdv_query_head_uses_key_length": [("      const size_t qhead = (size_t)bh * (size_t)Nq * (size_t)d;\n      const size_t khead = (size_t)bh * (size_t)Nk * (size_t)d;\n      const size_t rows",
                                         "      const size_t qhead = (size_t)bh * (size_t)Nk * (size_t)d;\n      const size_t khead = (size_t)bh * (size_t)Nk * (size_t)d;\n      const size_t rows")],
    "dq_keys_counted_with_query_length": [("dq_row(q + qhead, k + khead, v + khead, dout + qhead, Nk, d,",
                                           "dq_row(q + qhead, k + khead, v + khead, dout + qhead, Nk < Nq ? Nk : Nq, d,")],
    "dq_causal_excludes_diagonal": [("  const int64_t n_keys = causal ? i + 1 : N;\n  for (int64_t c = 0; c < d; ++c) dq[c] = 0.0;",
                                     "  const int64_t n_keys = causal ? i : N;\n  for (int64_t c = 0; c < d; ++c) dq[c] = 0.0;")],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    src = open(SRC).read()
    for old, new in MUTANTS[name]:
        assert old in src, "mutation anchor missing: %r" % old
        src = src.replace(old, new, 1)
    path = tmp_path / ("mutant_%s.c" % name)
    path.write_text(src)
    lib = oracle.open_bwd_oracle_library(oracle.compile_oracle(str(path), str(tmp_path / "m.so")))

    def grads(q, k, v, dout, causal, scale, qrows=None, krows=None):
        return oracle.attn_bwd_oracle(q, k, v, dout, causal=causal, scale=scale, qrows=qrows,
                                      krows=krows, lib=lib)

    failed = []
    for check in oracle_bwd_pins.ALL_CHECKS:
        try:
            check(grads)
        except AssertionError:
            failed.append(check.__name__)
            break
    assert failed, "planted mistake %r passed every pin" % name
