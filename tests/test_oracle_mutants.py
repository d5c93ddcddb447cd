"""Plant plausible mistakes in copies of the C oracle and check that some pin catches each.

The mutants are compiled from textual edits of ``oracle/la2_oracle.c`` into a
temporary directory; the real oracle is never touched.
"""
import os

import pytest

import oracle
from oracle import build as obuild
import pins

SRC = open(obuild.SRC).read()

# (name, original text, mutated text): each is a mistake someone could plausibly make.
MUTANTS = [
    ("no_decay_forward",
     "S[i * dv + j] = l * S[i * dv + j] + kt[i] * vt[j];\n            /* o_t",
     "S[i * dv + j] = S[i * dv + j] + kt[i] * vt[j];\n            /* o_t"),
    ("decay_on_current_token",
     "S[i * dv + j] = l * S[i * dv + j] + kt[i] * vt[j];\n            /* o_t",
     "S[i * dv + j] = l * (S[i * dv + j] + kt[i] * vt[j]);\n            /* o_t"),
    ("wrong_operand_readout",
     "acc += S[i * dv + j] * qt[i];",
     "acc += S[i * dv + j] * kt[i];"),
    ("reverse_state_uses_k",
     "R[i * dv + j] = l * R[i * dv + j] + qt[i] * gt[j];",
     "R[i * dv + j] = l * R[i * dv + j] + kt[i] * gt[j];"),
    ("dv_uses_q",
     "acc += R[i * dv + j] * kt[i];",
     "acc += R[i * dv + j] * qt[i];"),
    ("dk_sign",
     "acc += R[i * dv + j] * vt[j];",
     "acc -= R[i * dv + j] * vt[j];"),
    ("dq_forward_no_decay",
     "S[i * dv + j] = l * S[i * dv + j] + kt[i] * vt[j];\n            for (int64_t i = 0; i < d; ++i) {",
     "S[i * dv + j] = S[i * dv + j] + kt[i] * vt[j];\n            for (int64_t i = 0; i < d; ++i) {"),
    ("rows_exponent_off_by_one",
     "const double w = pow(lam, (double)(t - s)) * dot(q + t * d, k + s * d, d);",
     "const double w = pow(lam, (double)(t - s + 1)) * dot(q + t * d, k + s * d, d);"),
    ("rows_dk_wrong_vector",
     "const double wk = p * dot(dout + s * dv, v + t * dv, dv);",
     "const double wk = p * dot(dout + t * dv, v + s * dv, dv);"),
    ("state_in_transposed",
     "S[i * dv + j] = s_in[c * d * dv + i * dv + j];",
     "S[i * dv + j] = s_in[c * d * dv + j * d + i];"),
    ("state_out_before_last_step",
     "        if (s_out)\n            for (int64_t i = 0; i < d; ++i)",
     "        if (s_out && T > 0) { for (int64_t i = 0; i < d * dv; ++i) S[i] -= kc[(T - 1) * d + i / dv] * vc[(T - 1) * dv + i % dv]; }\n        if (s_out)\n            for (int64_t i = 0; i < d; ++i)"),
    ("normalized_denominator_no_decay",
     "z[i] = l * z[i] + pk[i];",
     "z[i] = z[i] + pk[i];"),
    ("normalized_feature_branch_swapped",
     "return x > 0.0 ? x + 1.0 : exp(x);",
     "return x > 0.0 ? exp(x) : x + 1.0;"),
    ("normalized_query_feature_skipped",
     "pq[i] = feature(qt[i], fmap);",
     "pq[i] = qt[i];"),
    ("dstate_in_missing_decay",
     "ds_in[c * d * dv + e] = l * R[e];",
     "ds_in[c * d * dv + e] = R[e];"),
    ("dstate_out_ignored",
     "                    R[e] += ds_out[c * d * dv + e];",
     "                    R[e] += 0.0 * ds_out[c * d * dv + e];"),
    ("backward_ignores_state_in",
     "            for (int64_t e = 0; e < d * dv; ++e)\n                S[e] = s_in[c * d * dv + e];",
     "            for (int64_t e = 0; e < d * dv; ++e)\n                S[e] = 0.0 * s_in[c * d * dv + e];"),
    ("normalized_backward_dden_sign",
     "dden[t] = -go / den;",
     "dden[t] = go / den;"),
    ("normalized_backward_no_feature_deriv",
     "dkc[t * d + i] = acc * feature_deriv(kc[t * d + i], fmap);",
     "dkc[t * d + i] = acc;"),
    ("normalized_backward_y_undecayed",
     "y[i] = l * y[i] + dden[t] * pqt[i];",
     "y[i] = y[i] + dden[t] * pqt[i];"),
    ("rows_skip_diagonal",
     "for (int64_t s = 0; s <= t; ++s) {\n            const double w = pow(lam, (double)(t - s)) * dot(q",
     "for (int64_t s = 0; s < t; ++s) {\n            const double w = pow(lam, (double)(t - s)) * dot(q"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    assert SRC.count(old) == 1, f"mutation site for {name} not unique"
    src = tmp_path / f"{name}.c"
    src.write_text(SRC.replace(old, new))
    lib = obuild.compile_oracle(str(src), str(tmp_path / f"{name}.so"))
    orc = oracle.load(lib)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
