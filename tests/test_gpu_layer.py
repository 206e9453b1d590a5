"""GPU parity of the linear-attention layer (la_layer_forward /
la_layer_backward) against the fp64 oracle layer (marked gpu).

Y, dX, dWqkv and dWo are compared element by element with the oracle fed the
same stored inputs: tensor-wide, and row by row (rows of Y and dX are tokens,
of the weight gradients their matrix rows; tests/parity_checks.py).  Tolerances: fp32 1e-5
(as for the attention alone); bf16 2e-2; fp16 2e-3.  Storage rounding enters
the layer at more points than the attention alone (the projected Q, K, V,
the merged O and Y forward; dO, dQ, dK, dV, dQKV and the three gradients
backward), about six roundings of at most 2^-9 (bf16) or 2^-12 (fp16)
relative each on the longest path, so the bf16 bound is the attention's and
the fp16 bound is twice the attention's.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from linear_attention_transformer_amd.inputs import make_layer_inputs
from tests import parity_checks as pc

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2, torch.float16: 2e-3}
DEV = "cuda:0"


def la():
    import linear_attention_transformer_amd as m
    m.load_library()
    return m


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().double().cpu().numpy()


def compare_layer(B, N, C, H, D, dtype, causal, seed=0):
    m = la()
    say("case layer B=%d N=%d C=%d H=%d D=%d %s causal=%d" % (B, N, C, H, D, dtype, causal))
    x, wqkv, wo, dy = make_layer_inputs(B, N, C, H, D, dtype=dtype, seed=seed, device=DEV)
    y, saved = m.layer_forward(x, wqkv, wo, H, causal)
    dx, dwqkv, dwo = m.layer_backward(x, wqkv, wo, dy, H, causal, saved=saved)
    torch.cuda.synchronize()
    a = [f64(t) for t in (x, wqkv, wo, dy)]
    y_r = oracle.layer_forward(*a[:3], H, D, causal)
    g_r = oracle.layer_backward(*a, H, D, causal)
    errs = []
    for name, got, ref in zip(("Y", "dX", "dWqkv", "dWo"), (y, dx, dwqkv, dwo), (y_r,) + g_r):
        g = f64(got)
        assert np.all(np.isfinite(g)), name
        errs.append((name, pc.metrics(g, ref, ref.shape[-1], floor=pc.row_floor(TOL[dtype]))))
    pc.check_all(errs, TOL[dtype], say)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_layer_parity(causal, dtype):
    compare_layer(2, 300, 96, 3, 32, dtype, causal, seed=1)


@pytest.mark.parametrize("causal", [False, True])
def test_layer_padded_head_size(causal):
    """D = 20 (padded to 32 inside the attention) and C not a multiple of 16."""
    compare_layer(2, 130, 40, 2, 20, torch.float32, causal, seed=2)


@pytest.mark.parametrize("causal", [False, True])
def test_layer_longer_sequence(causal):
    compare_layer(1, 2048, 256, 4, 64, torch.float32, causal, seed=3)


def test_layer_forward_without_saved_buffer_and_errors():
    m = la()
    x, wqkv, wo, dy = make_layer_inputs(1, 64, 32, 2, 16, device=DEV)
    y1, saved = m.layer_forward(x, wqkv, wo, 2)
    y2, none = m.layer_forward(x, wqkv, wo, 2, save=False)
    torch.cuda.synchronize()
    assert none is None and torch.equal(y1, y2)
    with pytest.raises(m.LAError) as e:
        m.layer_forward(x, wqkv, wo, 2, out=x)            # output aliases the input
    assert e.value.code == 6
    with pytest.raises(m.LAError) as e:
        m.layer_backward(x, wqkv, wo, dy, 2, saved=saved,
                         workspace=torch.empty(1024, dtype=torch.uint8, device=DEV))
    assert e.value.code == 5
