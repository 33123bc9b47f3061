"""The oracle's pins must catch plausible mistakes.

Each case copies oracle.c, plants one mistake (a transposed operand, a wrong
sign, index or comparison, a dropped term, a missing stop), builds the mutant
with gcc into a temporary directory and runs the fast pins of
test_oracle_pins.py against it.  At least one pin must fail for every mutant.
Everything runs on the CPU; the real oracle library is restored afterwards.
"""
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

MUTANTS = [
    ("accept test in the wrong direction",
     "if (!(u < r)) { j = i; break; }", "if (!(u > r)) { j = i; break; }"),
    ("no stop at the first rejection",
     "if (!(u < r)) { j = i; break; }", "if (!(u < r)) { j = i; }"),
    ("ratio inverted", "const double r = p / q;", "const double r = q / p;"),
    ("residual operands transposed",
     "w[k] = p - q > 0.0 ? p - q : 0.0;", "w[k] = q - p > 0.0 ? q - p : 0.0;"),
    ("residual without the clip at zero",
     "w[k] = p - q > 0.0 ? p - q : 0.0;", "w[k] = p - q;"),
    ("final draw from the previous target row",
     "const int64_t tj = trow0 + j;", "const int64_t tj = trow0 + (j > 0 ? j - 1 : 0);"),
    ("final draw uses the stopping position's uniform",
     "const double u = (double)uniforms[trow0 + gamma];",
     "const double u = (double)uniforms[trow0 + j];"),
    ("inverse CDF admits a zero-weight token",
     "if (C[k] > t) { tok = k; break; }", "if (C[k] >= t) { tok = k; break; }"),
    ("normaliser drops the first term",
     "  double s = 0.0;\n  for (int64_t k = 0; k < vocab; ++k) {",
     "  double s = 0.0;\n  for (int64_t k = 1; k < vocab; ++k) {"),
    ("temperature multiplies instead of divides",
     "return exp(load_logit(base, dtype, row * ld + k) / T - M) / s;",
     "return exp(load_logit(base, dtype, row * ld + k) * T - M) / s;"),
    ("target rows without the per-sequence offset",
     "const int64_t trow0 = (int64_t)cu_draft[b] + b;",
     "const int64_t trow0 = (int64_t)cu_draft[b];"),
    ("accepted count off by one",
     "out_num_accepted[b] = (int32_t)j;", "out_num_accepted[b] = (int32_t)(j + 1);"),
]

FAST_PINS = [
    (pins.test_row_softmax_matches_scipy, dict(dtype="f32", T=0.7)),
    (pins.test_row_softmax_closed_forms, {}),
    (pins.test_p_q_at_draft_tokens_match_scipy, {}),
    (pins.test_identical_rows_accept_every_draft, dict(seed=0)),
    (pins.test_one_hot_target_accepts_its_argmax, dict(neg=float("-inf"))),
    (pins.test_golden_hand_cases, {}),
    (pins.test_zero_weight_token_never_drawn, {}),
    (pins.test_gamma_zero_is_textbook_inverse_cdf, dict(dtype="bf16", T=0.7)),
    (pins.test_one_hot_draft_reduces_to_bernoulli_and_renormalised_p, {}),
    (pins.test_residual_sum_is_total_variation, {}),
    (pins.test_midpoint_quadrature_first_token_law, {}),
    (pins.test_exact_enumeration_output_law, {}),
    (pins.test_edge_cases, {}),
    (pins.test_tie_flags, {}),
]


def _build_mutant(tmp_path, old, new):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    assert src.count(old) == 1, f"mutation site not unique: {old!r}"
    path = tmp_path / "oracle_mutant.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fPIC",
                    "-shared", "-o", str(lib), str(path), "-lm"], check=True)
    return str(lib)


@pytest.mark.slow
@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, monkeypatch, name, old, new):
    lib = _build_mutant(tmp_path, old, new)
    monkeypatch.setattr(oracle, "LIB_PATH", lib)
    monkeypatch.setattr(oracle, "_lib", None)
    caught = []
    for fn, kw in FAST_PINS:
        try:
            fn(oracle, **kw)
        except (AssertionError, ValueError, IndexError):
            caught.append(fn.__name__)
    monkeypatch.setattr(oracle, "_lib", None)
    assert caught, f"no pin caught the mutant: {name}"
