"""The row and head checks of tests/parity_checks.py catch what one
tensor-wide relative L2 error lets through (CPU only).

A correct 16-bit result is modelled by rounding the oracle's fp64 result to
the storage type (which is what the GPU path's outputs are, up to fp32
rounding inside).  Mistakes are planted into copies of it: one wrong row per
head, one wrong head.  Each passes the tensor-wide bound and fails the new
ones; the rounded copy itself passes them all.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
from linear_attention_transformer_amd.inputs import as_f64_numpy, make_inputs
from tests import parity_checks as pc

TOL_BF16 = 2e-2


@functools.lru_cache(maxsize=2)
def _case(causal, B=4, H=16, N=4096, D=32):
    q, k, v, g = make_inputs(B, H, N, D, dtype=torch.bfloat16, seed=31)
    a = [as_f64_numpy(x) for x in (q, k, v, g)]
    o, _ = oracle.forward_state(*a[:3], causal)
    dq, dk, dv = oracle.backward_state(*a, causal)
    rounded = lambda r: torch.from_numpy(r).to(torch.bfloat16).double().numpy()  # noqa: E731
    return {"O": (rounded(o), o), "dQ": (rounded(dq), dq), "dK": (rounded(dk), dk),
            "dV": (rounded(dv), dv)}, B * H, D


@pytest.mark.parametrize("causal", [False, True])
def test_rounded_result_passes_every_check(causal):
    outs, heads, D = _case(causal)
    for name, (x, r) in outs.items():
        m = pc.metrics(x, r, D, heads, floor=pc.row_floor(TOL_BF16))
        assert pc.failures(m, TOL_BF16) == [], (name, m)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("name", ["O", "dQ", "dK", "dV"])
def test_one_wrong_row_per_head_is_caught(causal, name):
    """The last row of every head zeroed (non-causal) or replaced by the row
    before it scaled by 1.5 (causal, where the last rows are small)."""
    outs, heads, D = _case(causal)
    x, r = outs[name]
    bad = x.copy()    # 4096 rows per head: one wrong row moves rel_l2 by about 1/64
    if causal:
        bad[:, :, -1] = 1.5 * bad[:, :, -2]
    else:
        bad[:, :, -1] = 0.0
    m = pc.metrics(bad, r, D, heads, floor=pc.row_floor(TOL_BF16))
    assert m["rel_l2"] <= TOL_BF16, m          # the tensor-wide bound passes
    assert "row" in pc.failures(m, TOL_BF16), m
    assert m["row_at"] % r.shape[2] == r.shape[2] - 1


@pytest.mark.parametrize("causal", [False, True])
def test_one_wrong_head_is_caught(causal):
    outs, heads, D = _case(causal)
    x, r = outs["dK"]
    bad = x.copy()
    bad[2, 5] *= 1.1
    m = pc.metrics(bad, r, D, heads, floor=pc.row_floor(TOL_BF16))
    assert m["rel_l2"] <= TOL_BF16, m
    assert "head" in pc.failures(m, TOL_BF16), m


def test_den_is_checked_element_by_element():
    """den is one value per row: one denominator off by 5% in a sequence of
    1024 fails against its own value, not against the tensor's scale."""
    q, k, v, _ = make_inputs(1, 2, 1024, 32, seed=3)
    a = [as_f64_numpy(x) for x in (q, k, v)]
    _, den = oracle.forward_state(*a, True)
    bad = den.copy()
    bad[0, 1, 3] *= 1.05
    m = pc.metrics(bad, den, 1, 2, floor=0.0)
    assert m["rel_l2"] <= TOL_BF16
    assert "row" in pc.failures(m, TOL_BF16)


def test_vanishing_reference_uses_the_given_scale():
    """dQ of one-token sequences is exactly zero: errors are then measured
    against the scale passed in, not divided by zero."""
    r = np.zeros((1, 2, 1, 8))
    x = np.full_like(r, 1e-9)
    m = pc.metrics(x, r, 8, 2, scale=1.0)
    assert np.isfinite(m["row"]) and pc.failures(m, 1e-5) == []
    m = pc.metrics(x + 1e-3, r, 8, 2, scale=1.0)
    assert "row" in pc.failures(m, 1e-5)
