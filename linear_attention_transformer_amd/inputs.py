"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module draws random numbers and nothing else: it holds none of the
attention arithmetic, so the oracle and the HIP path can both be fed from it
without sharing code.

Recipe (the workload shapes of Figures 2 and 3 on the sciencestack.ai page of
"Transformer Based Linear Attention with Optimized GPU Kernel Implementation":
B = 4, H = 16, D = 128 with an N sweep, and N = 4096 with a D sweep):

* Q, K, V, dO are drawn in that order from ONE generator seeded with ``seed``,
  each ``torch.randn([B, H, N, D])`` in fp32, i.i.d. standard normal;
* Q, K, V are divided by sqrt(D); dO is left unscaled;
* storage dtypes other than fp32 are produced by ``.to(dtype)`` (round to
  nearest even), so a consumer that wants the exact stored values upcasts the
  returned tensors;
* layout [B, H, N, D], contiguous.
"""
from __future__ import annotations

import math

import torch

# above this many elements per tensor the draw happens on the GPU
DEVICE_DRAW_THRESHOLD = 1 << 26


def make_inputs(B: int, H: int, N: int, D: int, *, dtype=torch.float32,
                seed: int = 0, device="cpu", draw_device=None):
    """Return (q, k, v, do) on ``device`` with storage ``dtype``."""
    shape = (B, H, N, D)
    numel = B * H * N * D
    if draw_device is None:
        draw_device = device if numel > DEVICE_DRAW_THRESHOLD else "cpu"
    gen = torch.Generator(device=draw_device)
    gen.manual_seed(seed)
    scale = 1.0 / math.sqrt(D)
    out = []
    for i in range(4):
        x = torch.randn(shape, generator=gen, device=draw_device,
                        dtype=torch.float32)
        if i < 3:
            x.mul_(scale)
        out.append(x.to(device=device, dtype=dtype).contiguous())
    return tuple(out)


def as_f64_numpy(t: torch.Tensor):
    """Exact fp64 copy of a stored tensor, as a numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def make_layer_inputs(B: int, N: int, C: int, H: int, D: int, *, dtype=torch.float32,
                      seed: int = 0, device="cpu"):
    """Return (x, wqkv, wo, dy) for one attention layer, drawn in that order
    from one CPU generator seeded with ``seed`` (fp32 randn, then scaled):

    * x [B, N, C] and dy [B, N, C]: standard normal;
    * wqkv [C, 3*H*D]: the query and key columns scaled by 1/sqrt(C*D), so
      that queries and keys have the N(0, 1/D) entries of the head-batch
      recipe above; the value columns by 1/sqrt(C);
    * wo [H*D, C]: scaled by 1/sqrt(H*D);

    then ``.to(dtype)`` (round to nearest even) on ``device``."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    HD = H * D
    x = torch.randn((B, N, C), generator=gen)
    wqkv = torch.randn((C, 3 * HD), generator=gen)
    wqkv[:, :2 * HD] /= math.sqrt(C * D)
    wqkv[:, 2 * HD:] /= math.sqrt(C)
    wo = torch.randn((HD, C), generator=gen) / math.sqrt(HD)
    dy = torch.randn((B, N, C), generator=gen)
    return tuple(t.to(device=device, dtype=dtype).contiguous() for t in (x, wqkv, wo, dy))
