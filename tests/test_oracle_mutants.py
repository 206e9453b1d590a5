"""Plant plausible mistakes in a copy of the oracle source (CPU only) and
check that the pins catch every one of them.

Each mutant is compiled from a modified copy of oracle/la_oracle.c into a
temporary library; the pins of test_oracle_pins.py are then run against it
and at least one must fail.  The real oracle is never modified.
"""
import pytest

import oracle
from tests import test_oracle_carry as carry
from tests import test_oracle_pins as pins

# (name, text in la_oracle.c, replacement)
MUTANTS = [
    ("drop constant term", "return 1.0 + dot;", "return dot;"),
    ("drop count in state denominator", "double den = n + dotv(q, z, D);",
     "double den = dotv(q, z, D);"),
    ("transposed state in apply", "num += q[d] * S[d * D + e];",
     "num += q[d] * S[e * D + d];"),
    ("constant term missing from state numerator", "double num = u[e];",
     "double num = 0.0;"),
    ("sign of c_i z term", "dq[d] = y - c * z[d];", "dq[d] = y + c * z[d];"),
    ("transposed S in dq", "y += S[d * D + e] * a[e];",
     "y += S[e * D + d] * a[e];"),
    ("causal mask excludes diagonal", "return causal ? i + 1 : N;",
     "return causal ? (i > 0 ? i : 1) : N;"),
    ("reverse sweep misses the diagonal",
     "            grad_state_add(R, r, t, q + j * D, A + j * D, C[j], D);\n"
     "            grad_state_apply(R, r, t, k + j * D, v + j * D, dk + j * D,\n"
     "                             dv + j * D, D);",
     "            grad_state_apply(R, r, t, k + j * D, v + j * D, dk + j * D,\n"
     "                             dv + j * D, D);\n"
     "            grad_state_add(R, r, t, q + j * D, A + j * D, C[j], D);"),
    ("dv misses the t term", "double s = t[e];", "double s = 0.0;"),
    ("dk misses the r term", "dk[d] = s - r[d];", "dk[d] = s;"),
    ("direct dv uses w of the wrong pair",
     "double w = sim(q + i * D, k + j * D, D);\n            for (int64_t d = 0; d < D; ++d) {",
     "double w = sim(q + j * D, k + i * D, D);\n            for (int64_t d = 0; d < D; ++d) {"),
    ("c_i uses g instead of a", "double c = dotv(a, o + i * D, D);",
     "double c = dotv(g + i * D, o + i * D, D);"),
    ("carried count left out of the non-causal denominator",
     "state_apply(S, z, u, n0 + (double)N,", "state_apply(S, z, u, (double)N,"),
    ("gradient carry ignored", "record_load(grec_in, R, r, t, D);", ""),
    ("carried record stored with z and u swapped",
     "memcpy(rec + D * D + D, u, sizeof(double) * (size_t)D);",
     "memcpy(rec + D * D + D, z, sizeof(double) * (size_t)D);"),
    ("causal count off by one", "(double)(i + 1), q + i * D,\n                                    o + i * D, D);",
     "(double)(i), q + i * D,\n                                    o + i * D, D);"),
]


def _pin_cases():
    cases = []
    for form in pins.FORMS:
        for causal in (False, True):
            cases.append((pins.test_worked_examples, dict(form=form, causal=causal)))
            cases.append((pins.test_fd_directional, dict(form=form, causal=causal)))
            cases.append((pins.test_reparametrisation, dict(form=form, causal=causal)))
            cases.append((pins.test_constant_values_give_constant_output,
                          dict(form=form, causal=causal)))
    for causal in (False, True):
        cases.append((pins.test_direct_matches_state,
                      dict(shape=(1, 2, 16, 4), causal=causal)))
        cases.append((pins.test_autograd_gradients,
                      dict(shape=(1, 3, 7, 5), causal=causal)))
        cases.append((pins.test_first_order_agreement_with_softmax, dict(causal=causal)))
        cases.append((carry.test_pieces_forward_match_whole_sequence, dict(causal=causal)))
        cases.append((carry.test_pieces_backward_match_whole_sequence, dict(causal=causal)))
        cases.append((carry.test_gradient_record_is_derivative_of_carried_state,
                      dict(causal=causal)))
    return cases


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = oracle.source_text()
    assert src.count(old) == 1, "mutation site not found uniquely: %s" % name
    variant = oracle.build_variant(src.replace(old, new), str(tmp_path))
    caught = []
    for fn, kw in _pin_cases():
        try:
            fn(variant, **kw)
        except (AssertionError, FloatingPointError, ValueError):
            caught.append(fn.__name__)
    assert caught, "no pin caught the mutant '%s'" % name
