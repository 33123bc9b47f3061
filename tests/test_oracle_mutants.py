"""The oracle's pins must catch plausible mistakes.

Each case copies oracle.c, plants one mistake (a transposed operand, a wrong
sign, index or comparison, a dropped term, a missing stop) inside one
function, builds the mutant with gcc into a temporary directory and runs that
function's fast pins (test_oracle_pins.py for the sampled verify,
test_oracle_pins_modes.py for greedy and point-mass drafts) against it.  At
least one pin must fail for every mutant.  Everything runs on the CPU; the
real oracle library is restored afterwards.
"""
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins
from tests import test_oracle_pins_modes as mpins
from tests import test_oracle_pins_tree as tpins
from tests import test_oracle_pins_precision as ppins

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
     "  double err = 0.0;\n  for (int64_t k = 0; k < vocab; ++k) {",
     "  double err = 0.0;\n  for (int64_t k = 1; k < vocab; ++k) {"),
    ("temperature multiplies instead of divides",
     "const double z = load_logit(base, dtype, row * ld + k) / T;",
     "const double z = load_logit(base, dtype, row * ld + k) * T;"),
    ("compensated sum drops its correction",
     "static double csum_value(const csum *a) { return a->hi + a->lo; }",
     "static double csum_value(const csum *a) { return a->hi; }"),
    ("target rows without the per-sequence offset",
     "const int64_t trow0 = (int64_t)cu_draft[b] + b;",
     "const int64_t trow0 = (int64_t)cu_draft[b];"),
    ("accepted count off by one",
     "out_num_accepted[b] = (int32_t)j;", "out_num_accepted[b] = (int32_t)(j + 1);"),
]

SAMPLED = "int oracle_verify("
GREEDY = "int oracle_verify_greedy("
POINT = "int oracle_verify_onehot("

MODE_MUTANTS = [
    ("greedy: ties go to the highest id", None,
     "if (v > bv) { bv = v; best = k; }", "if (v >= bv) { bv = v; best = k; }"),
    ("greedy: no stop at the first mismatch", GREEDY,
     "{ j = i; break; }", "{ j = i; }"),
    ("greedy: mismatch emits the previous row's argmax", GREEDY,
     "else if (i == j) v = (int32_t)row_argmax(target_logits, dtype, trow0 + j, ld, vocab);",
     "else if (i == j) v = (int32_t)row_argmax(target_logits, dtype, trow0 + (j > 0 ? j - 1 : 0), ld, vocab);"),
    ("greedy: target rows without the per-sequence offset", GREEDY,
     "const int64_t trow0 = (int64_t)cu_draft[b] + b;", "const int64_t trow0 = (int64_t)cu_draft[b];"),
    ("point: rejected token kept in the residual", POINT,
     "const double q = (k == draft_tokens[drow0 + j]) ? 1.0 : 0.0;", "const double q = 0.0;"),
    ("point: accept test not strict", POINT,
     "if (!(u < px)) { j = i; break; }", "if (!(u <= px)) { j = i; break; }"),
    ("point: accept test against 1 - p(x)", POINT,
     "if (!(u < px)) { j = i; break; }", "if (!(u < 1.0 - px)) { j = i; break; }"),
    ("point: residual drawn from the next row", POINT,
     "const int64_t tj = trow0 + j;", "const int64_t tj = trow0 + (j < gamma ? j + 1 : j);"),
    ("point: final draw uses the stopping position's uniform", POINT,
     "const double u = (double)uniforms[trow0 + gamma];",
     "const double u = (double)uniforms[trow0 + j];"),
]

TGREEDY = "int oracle_verify_tree_greedy("
TPOINT = "int oracle_verify_tree_point("

TREE_MUTANTS = [
    ("tree greedy: the last matching child", TGREEDY,
     "if (parent[g0 + n] == cur && tokens[g0 + n] == a) { next = n; break; }",
     "if (parent[g0 + n] == cur && tokens[g0 + n] == a) { next = n; }"),
    ("tree greedy: children of the root at every level", TGREEDY,
     "if (parent[g0 + n] == cur && tokens[g0 + n] == a)",
     "if (parent[g0 + n] == 0 && tokens[g0 + n] == a)"),
    ("tree point: no renormalisation after a rejection", TPOINT,
     "r = p[x] / csum_value(&rest);", "r = p[x];"),
    ("tree point: rejected tokens kept in the final draw", TPOINT,
     "w[k] = removed[k] ? 0.0 : p[k];", "w[k] = p[k];"),
    ("tree point: a repeated token tested again", TPOINT,
     "r = 0.0;                     /* already rejected: p'(x) = 0 */",
     "r = p[x];"),
    ("tree point: final draw with the stopping node's uniform", TPOINT,
     "const double u = (double)uniforms[g0];", "const double u = (double)uniforms[g0 + cur];"),
    ("tree point: removals carried to the next level", TPOINT,
     "if (parent[g0 + n] == cur) removed[tokens[g0 + n]] = 0;",
     "if (parent[g0 + n] == cur && 0) removed[tokens[g0 + n]] = 0;"),
]

TREE_PINS = [
    (tpins.test_tree_golden_cases, {}),
    (tpins.test_chain_trees_reduce_to_chain_verifiers, dict(dtype="bf16")),
    (tpins.test_greedy_path_follows_numpy_argmax, {}),
    (tpins.test_point_tree_output_law, {}),
]

MODE_PINS = [
    (mpins.test_greedy_golden_cases, {}),
    (mpins.test_greedy_argmax_is_numpy_first_occurrence, dict(dtype="bf16")),
    (mpins.test_greedy_is_the_zero_temperature_limit_of_sampled_verify, {}),
    (mpins.test_point_draft_golden_cases, {}),
    (mpins.test_point_drafts_equal_sampled_verify_with_point_mass_q, dict(dtype="bf16", T=0.7)),
    (mpins.test_point_draft_accept_threshold_is_p_of_x, {}),
    (mpins.test_point_draft_output_law_by_grid_count, {}),
    (mpins.test_point_draft_edge_cases, {}),
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
    (ppins.test_compensated_normaliser_keeps_sub_ulp_tail, {}),
]


def _build_mutant(tmp_path, old, new, scope=SAMPLED):
    """Replace `old` (which must occur exactly once in the body of the
    function that starts with `scope`) by `new`."""
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    if scope is None:                       # a site unique in the whole file
        assert src.count(old) == 1, f"mutation site not unique: {old!r}"
        path = tmp_path / "oracle_mutant.c"
        path.write_text(src.replace(old, new))
        return _compile(tmp_path, path)
    start = src.index(scope)
    end = src.find("\nint oracle_", start + 1)
    end = len(src) if end < 0 else end
    body = src[start:end]
    assert body.count(old) == 1, f"mutation site not unique in {scope}: {old!r}"
    path = tmp_path / "oracle_mutant.c"
    path.write_text(src[:start] + body.replace(old, new) + src[end:])
    return _compile(tmp_path, path)


def _compile(tmp_path, path):
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fPIC",
                    "-shared", "-o", str(lib), str(path), "-lm"], check=True)
    return str(lib)


@pytest.mark.slow
@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, monkeypatch, name, old, new):
    # helper-function sites are unique in the file; sites inside the sampled
    # verify function are looked up in its body
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    lib = _build_mutant(tmp_path, old, new, None if src.count(old) == 1 else SAMPLED)
    _expect_caught(monkeypatch, lib, FAST_PINS, name)


def _expect_caught(monkeypatch, lib, pin_list, name):
    monkeypatch.setattr(oracle, "LIB_PATH", lib)
    monkeypatch.setattr(oracle, "_lib", None)
    caught = []
    for fn, kw in pin_list:
        try:
            fn(oracle, **kw)
        except (AssertionError, ValueError, IndexError):
            caught.append(fn.__name__)
    monkeypatch.setattr(oracle, "_lib", None)
    assert caught, f"no pin caught the mutant: {name}"


@pytest.mark.slow
@pytest.mark.parametrize("name,scope,old,new", MODE_MUTANTS, ids=[m[0] for m in MODE_MUTANTS])
def test_mode_pins_catch_mutant(tmp_path, monkeypatch, name, scope, old, new):
    lib = _build_mutant(tmp_path, old, new, scope)
    _expect_caught(monkeypatch, lib, MODE_PINS, name)


@pytest.mark.slow
@pytest.mark.parametrize("name,scope,old,new", TREE_MUTANTS, ids=[m[0] for m in TREE_MUTANTS])
def test_tree_pins_catch_mutant(tmp_path, monkeypatch, name, scope, old, new):
    lib = _build_mutant(tmp_path, old, new, scope)
    _expect_caught(monkeypatch, lib, TREE_PINS, name)
