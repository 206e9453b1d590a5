"""Pins of the oracle's linear-attention layer (CPU only).

The layer oracle composes fp64 matrix products with the attention oracle's
state form and a hand-written chain rule.  It is pinned against torch
autograd through a layer built from the O(N^2) pairwise attention
definition, and against central finite differences of its own forward.
"""
import math

import numpy as np
import pytest
import torch

from linear_attention_transformer_amd.inputs import make_layer_inputs


def _torch_layer(x, wqkv, wo, H, D, causal):
    """The layer written with the pairwise attention definition in torch."""
    B, N, _ = x.shape
    HD = H * D
    qkv = x @ wqkv
    q, k, v = (qkv[..., j * HD:(j + 1) * HD].reshape(B, N, H, D).transpose(1, 2)
               for j in range(3))
    w = 1.0 + q @ k.transpose(-1, -2)
    if causal:
        w = w * torch.tril(torch.ones(N, N, dtype=w.dtype))
    o = (w @ v) / w.sum(-1, keepdim=True)
    return o.transpose(1, 2).reshape(B, N, HD) @ wo


def _inputs(B, N, C, H, D, seed=2):
    return [t.double().numpy() for t in make_layer_inputs(B, N, C, H, D, seed=seed)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 9, 7, 2, 3), (1, 16, 12, 3, 4)])
def test_layer_matches_autograd_of_pairwise_definition(oracle_mod, shape, causal):
    """Catches a transposed projection, heads split or merged in the wrong
    order, and a wrong chain rule through either product."""
    B, N, C, H, D = shape
    x, wqkv, wo, dy = _inputs(B, N, C, H, D)
    y = oracle_mod.layer_forward(x, wqkv, wo, H, D, causal)
    t = [torch.tensor(a, requires_grad=True) for a in (x, wqkv, wo)]
    yt = _torch_layer(*t, H, D, causal)
    assert np.allclose(y, yt.detach().numpy(), rtol=1e-12, atol=1e-12)
    (yt * torch.tensor(dy)).sum().backward()
    got = oracle_mod.layer_backward(x, wqkv, wo, dy, H, D, causal)
    for g, a in zip(got, t):
        ref = a.grad.numpy()
        assert np.linalg.norm(g - ref) <= 1e-11 * max(np.linalg.norm(ref), 1.0)


@pytest.mark.parametrize("causal", [False, True])
def test_layer_gradients_by_finite_differences(oracle_mod, causal):
    B, N, C, H, D = 1, 8, 6, 2, 4
    x, wqkv, wo, dy = _inputs(B, N, C, H, D, seed=5)
    grads = oracle_mod.layer_backward(x, wqkv, wo, dy, H, D, causal)
    rng = np.random.default_rng(3)
    args = [x, wqkv, wo]
    for i in range(3):
        d = rng.standard_normal(args[i].shape)
        eps = 1e-6

        def loss(s):
            a = list(args)
            a[i] = args[i] + s * d
            return float(np.sum(dy * oracle_mod.layer_forward(*a, H, D, causal)))

        fd = (loss(eps) - loss(-eps)) / (2 * eps)
        an = float(np.sum(d * grads[i]))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (i, fd, an)


def test_layer_input_recipe_scales():
    """Queries and keys from the layer recipe have about N(0, 1/D) entries,
    as in the head-batch recipe; values and outputs about unit scale."""
    B, N, C, H, D = 2, 256, 512, 4, 64
    x, wqkv, wo, _ = make_layer_inputs(B, N, C, H, D, seed=1)
    qkv = x @ wqkv
    HD = H * D
    for j, want in ((0, 1 / D), (1, 1 / D), (2, 1.0)):
        var = float(qkv[..., j * HD:(j + 1) * HD].var())
        assert abs(var / want - 1) < 0.1, (j, var, want)
    assert abs(float(wo.var()) * HD - 1) < 0.1
    assert math.isclose(float(x.var()), 1.0, rel_tol=0.05)
