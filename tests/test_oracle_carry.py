"""Pins of the oracle's carried-state evaluation (CPU only).

A sequence cut into pieces and evaluated piece by piece, each piece starting
from the record its neighbours leave, must give exactly the rows of the whole
sequence.  The whole sequence is evaluated by the O(N^2) pairwise definition,
so these pins do not lean on the state form they check.  The gradient record
a piece returns is pinned as the derivative of the piece's loss with respect
to the record it was given (central finite differences).
"""
import math

import numpy as np
import pytest

PIECES = (5, 9, 7)   # a ragged cut of N = 21


def _inputs(B=2, H=2, D=6, seed=3):
    rng = np.random.default_rng(seed)
    N = sum(PIECES)
    shape = (B, H, N, D)
    q, k, v = (rng.standard_normal(shape) / math.sqrt(D) for _ in range(3))
    g = rng.standard_normal(shape)
    return q, k, v, g


def _cuts():
    out, s = [], 0
    for n in PIECES:
        out.append(slice(s, s + n))
        s += n
    return out


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1.0)


def _forward_records(oracle, q, k, v, causal):
    """(rec_in, n0) of every piece."""
    cuts = _cuts()
    N = q.shape[2]
    if causal:
        out, rec, n0 = [], None, 0
        for c in cuts:
            out.append((rec, n0))
            _, _, rec = oracle.forward_carry(q[:, :, c], k[:, :, c], v[:, :, c], True, rec, n0)
            n0 += c.stop - c.start
        return out
    own = [oracle.forward_carry(q[:, :, c], k[:, :, c], v[:, :, c], False)[2] for c in cuts]
    return [(sum(r for j, r in enumerate(own) if j != i), N - (c.stop - c.start))
            for i, c in enumerate(cuts)]


@pytest.mark.parametrize("causal", [False, True])
def test_pieces_forward_match_whole_sequence(oracle_mod, causal):
    """Catches a dropped or doubled carried state, a carried count that is
    left out of the denominator, and a record with S transposed or z and u
    swapped (the pieces would then disagree with the pairwise definition)."""
    q, k, v, _ = _inputs()
    o_ref, den_ref = oracle_mod.forward_direct(q, k, v, causal)
    for c, (rec, n0) in zip(_cuts(), _forward_records(oracle_mod, q, k, v, causal)):
        o, den, _ = oracle_mod.forward_carry(q[:, :, c], k[:, :, c], v[:, :, c], causal, rec, n0)
        assert _rel(o, o_ref[:, :, c]) < 1e-12
        assert _rel(den, den_ref[:, :, c]) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_pieces_backward_match_whole_sequence(oracle_mod, causal):
    """Causal: pieces in reverse order, each handing its gradient record to
    the piece before it.  Non-causal: every piece first forms its own rows'
    record, then each piece takes the sum of the others'.  Catches a gradient
    carry that is dropped, or that reaches dK and dV with the wrong sign."""
    q, k, v, g = _inputs()
    dq_ref, dk_ref, dv_ref = oracle_mod.backward_direct(q, k, v, g, causal)
    cuts = _cuts()
    fr = _forward_records(oracle_mod, q, k, v, causal)
    sl = lambda x, c: x[:, :, c]  # noqa: E731
    got = [None] * len(cuts)
    if causal:
        grec = None
        for i in reversed(range(len(cuts))):
            c, (rec, n0) = cuts[i], fr[i]
            *grads, grec = oracle_mod.backward_carry(sl(q, c), sl(k, c), sl(v, c), sl(g, c),
                                                     True, rec, n0, grec)
            got[i] = grads
    else:
        own = [oracle_mod.backward_carry(sl(q, c), sl(k, c), sl(v, c), sl(g, c), False,
                                         rec, n0)[3] for c, (rec, n0) in zip(cuts, fr)]
        for i, (c, (rec, n0)) in enumerate(zip(cuts, fr)):
            others = sum(r for j, r in enumerate(own) if j != i)
            *grads, _ = oracle_mod.backward_carry(sl(q, c), sl(k, c), sl(v, c), sl(g, c),
                                                  False, rec, n0, others)
            got[i] = grads
    for c, (dq, dk, dv) in zip(cuts, got):
        assert _rel(dq, sl(dq_ref, c)) < 1e-11
        assert _rel(dk, sl(dk_ref, c)) < 1e-11
        assert _rel(dv, sl(dv_ref, c)) < 1e-11


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_record_is_derivative_of_carried_state(oracle_mod, causal):
    """For L = sum_i g_i . o_i over a piece, the gradient record it returns
    (given no gradient carry) is [dL/dS | -dL/dz | dL/du] at the carried
    record.  Checked by central differences along random directions; catches
    a wrong sign of r, a transposed R, and a missing t."""
    B, H, N, D = 1, 2, 6, 4
    rng = np.random.default_rng(11)
    mk = lambda n, s=1.0: rng.standard_normal((B, H, n, D)) * s  # noqa: E731
    kp, vp = mk(9, 1 / math.sqrt(D)), mk(9, 1 / math.sqrt(D))
    _, _, rec = oracle_mod.forward_carry(mk(9), kp, vp, causal)   # a plausible record
    q, k, v, g = mk(N, 1 / math.sqrt(D)), mk(N, 1 / math.sqrt(D)), mk(N, 1 / math.sqrt(D)), mk(N)
    *_, grec = oracle_mod.backward_carry(q, k, v, g, causal, rec, 9)
    DD = D * D
    sign = np.concatenate([np.ones(DD), -np.ones(D), np.ones(D)])

    def loss(r):
        o, _, _ = oracle_mod.forward_carry(q, k, v, causal, r, 9)
        return float(np.sum(g * o))

    for trial in range(4):
        d = rng.standard_normal(rec.shape)
        eps = 1e-6
        fd = (loss(rec + eps * d) - loss(rec - eps * d)) / (2 * eps)
        an = float(np.sum(d * grec * sign))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (trial, fd, an)


@pytest.mark.parametrize("causal", [False, True])
def test_carry_edge_cases(oracle_mod, causal):
    """No carry equals the plain state form; an empty piece hands its record
    through unchanged, forward and backward."""
    q, k, v, g = _inputs(B=1, H=2, D=5)
    o0, d0 = oracle_mod.forward_state(q, k, v, causal)
    o1, d1, rec = oracle_mod.forward_carry(q, k, v, causal)
    assert np.array_equal(o0, o1) and np.array_equal(d0, d1)
    b0 = oracle_mod.backward_state(q, k, v, g, causal)
    *b1, grec = oracle_mod.backward_carry(q, k, v, g, causal)
    for a, b in zip(b0, b1):
        assert np.array_equal(a, b)
    e = q[:, :, :0]
    _, _, rec2 = oracle_mod.forward_carry(e, e, e, causal, rec, 21)
    assert np.array_equal(rec2, rec)
    *_, grec2 = oracle_mod.backward_carry(e, e, e, e, causal, rec, 21, grec)
    assert np.array_equal(grec2, grec)


def test_token_by_token_matches_whole_sequence(oracle_mod):
    """The recurrent decode reading: one-token causal pieces, each starting
    from the record the previous token left, give the causal rows of the
    pairwise definition.  Catches a decode step that counts the new token
    twice or not at all, or applies the state before adding the token."""
    q, k, v, _ = _inputs(B=1, H=2, D=4)
    o_ref, den_ref = oracle_mod.forward_direct(q, k, v, True)
    rec = None
    for i in range(q.shape[2]):
        c = slice(i, i + 1)
        o, den, rec = oracle_mod.forward_carry(q[:, :, c], k[:, :, c], v[:, :, c], True,
                                               rec, i)
        assert _rel(o, o_ref[:, :, c]) < 1e-12
        assert _rel(den, den_ref[:, :, c]) < 1e-12
