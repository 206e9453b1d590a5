"""The arithmetic behind the split products (CPU only): an fp32 value is the
exact sum of three bf16 terms taken by successive round-to-nearest, and the
six term products kept by the kernels (all but mid.lo, lo.mid, lo.lo) give
the product to within about 2^-22 of its size, below what the fp32
accumulation adds."""
import numpy as np
import torch


def _split3(x):
    hi = x.to(torch.bfloat16).to(torch.float32)
    r = x - hi                       # exact in fp32
    mid = r.to(torch.bfloat16).to(torch.float32)
    lo = (r - mid).to(torch.bfloat16).to(torch.float32)
    return hi, mid, lo


def test_three_bf16_terms_are_exact():
    g = torch.Generator().manual_seed(0)
    x = torch.randn(1 << 20, generator=g) * torch.exp2(torch.randint(-60, 60, (1 << 20,),
                                                                     generator=g).float())
    x = torch.cat([x, torch.tensor([1.0, -1.0, 3.0e-30, 1.0 + 2.0 ** -23, -(2.0 - 2.0 ** -23)])])
    hi, mid, lo = _split3(x)
    s = hi.double() + mid.double() + lo.double()
    assert torch.equal(s, x.double())


def test_six_term_products_within_fp32_rounding():
    g = torch.Generator().manual_seed(1)
    a = torch.randn(1 << 18, generator=g)
    b = torch.randn(1 << 18, generator=g)
    a1, a2, a3 = (t.double() for t in _split3(a))
    b1, b2, b3 = (t.double() for t in _split3(b))
    kept = a2 * b2 + a1 * b3 + a3 * b1 + a1 * b2 + a2 * b1 + a1 * b1
    exact = a.double() * b.double()
    rel = ((kept - exact).abs() / exact.abs().clamp_min(1e-300)).max().item()
    assert rel < 2.0 ** -21, rel
    # every term product is exact in fp32 (8 + 8 significant bits)
    for p in (a1 * b1, a2 * b3, a3 * b2):
        assert torch.equal(p, p.float().double())
    assert np.isfinite(rel)
