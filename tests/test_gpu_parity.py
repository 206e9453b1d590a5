"""GPU parity of the HIP library against the fp64 oracle (marked gpu).

Every case draws seeded inputs from the shared generator, runs the forward
and backward through the C ABI on cuda:0, and compares O, den, dQ, dK, dV
element by element (relative L2 per tensor) with the oracle fed the same
stored values.  Tolerances: fp32 storage 1e-5; bf16 storage (fp32
arithmetic, bf16 outputs) 2e-2; fp16 storage (fp32 arithmetic, fp16
outputs) 1e-3, from the fp16 rounding of the outputs (unit roundoff
2^-11 = 4.9e-4, relative L2 about 3e-4 for uniformly spread rounding).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from linear_attention_transformer_amd.inputs import as_f64_numpy, make_inputs

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2, torch.float16: 1e-3}
DEV = "cuda:0"


def la():
    import linear_attention_transformer_amd as m
    m.load_library()
    return m


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_l2(x, ref):
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-30))


def run_la(q, k, v, g, causal):
    m = la()
    o, den, st = m.forward(q, k, v, causal, return_den=True, save_state=True)
    dq, dk, dv = m.backward(q, k, v, g, causal, state=st)
    torch.cuda.synchronize()
    return o, den, dq, dk, dv


def compare(B, H, N, D, dtype, causal, heads=None, seed=0, lin_gate=True):
    """Run the HIP path on the full problem; check `heads` (all if None)."""
    say("case B=%d H=%d N=%d D=%d %s causal=%d seed=%d" % (B, H, N, D, dtype, causal, seed))
    q, k, v, g = make_inputs(B, H, N, D, dtype=dtype, seed=seed, device=DEV)
    got = run_la(q, k, v, g, causal)
    if heads is None:
        sel = lambda t: t
    else:
        idx = torch.tensor(heads, device=DEV)
        sel = lambda t: t.reshape(B * H, *t.shape[2:]).index_select(0, idx).unsqueeze(0)
    a = [as_f64_numpy(sel(x)) for x in (q, k, v, g)]
    o_ref, den_ref = oracle.forward_state(a[0], a[1], a[2], causal)
    refs = (o_ref, den_ref) + tuple(oracle.backward_state(*a, causal))
    tol = TOL[dtype]
    errs = {}
    # dQ and dK vanish in exact arithmetic when every row sees one token
    # (N = 1); their error is then measured against the gradient scale of
    # the same loss, ||dV|| (never zero: its rows sum to those of dO).
    gscale = np.linalg.norm(refs[4])
    for name, x, r in zip(("O", "den", "dQ", "dK", "dV"), got, refs):
        xs = as_f64_numpy(sel(x)).reshape(r.shape)
        assert np.all(np.isfinite(xs)), name
        den = max(np.linalg.norm(r), gscale if name in ("dQ", "dK") and N == 1 else 0.0)
        errs[name] = float(np.linalg.norm(xs - r) / max(den, 1e-30))
    say("  rel-L2 " + " ".join("%s=%.2e" % kv for kv in errs.items()))
    for name, e in errs.items():
        assert e <= tol, (name, e, tol)
    if dtype == torch.float32 and lin_gate and N > 1:
        # the linear term alone: O - O(Q=0) against the oracle's
        o0_ref, _ = oracle.forward_state(0 * a[0], a[1], a[2], causal)
        lin = as_f64_numpy(sel(got[0])).reshape(o_ref.shape) - o0_ref
        e = rel_l2(lin, o_ref - o0_ref)
        say("  linear-term rel-L2 %.2e" % e)
        assert e <= 1e-4
    return got


# ------------------------------------------------------------ small sizes
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_tiny_head(causal, dtype):
    """B=1, H=2, N=64, D=16 (the tiny workload)."""
    compare(1, 2, 64, 16, dtype, causal)


@pytest.mark.parametrize("D", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("N", [1, 17, 200, 1000])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_fp32(D, N, causal):
    """Lengths that are not multiples of any chunk, over every head size."""
    compare(1, 2, N, D, torch.float32, causal, seed=N + D)


@pytest.mark.parametrize("D", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_bf16(D, causal):
    compare(2, 1, 777, D, torch.bfloat16, causal, seed=3)


@pytest.mark.parametrize("D", [1, 6, 20, 48, 100, 200])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_generic_head_sizes(D, causal, dtype):
    """Head sizes between the native ones (D = 6 is the Figure 1 shape),
    padded to the next native size inside the library."""
    compare(2, 2, 333, D, dtype, causal, seed=D + 40)


@pytest.mark.parametrize("D", [6, 16, 32, 64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_fp16_storage(D, causal):
    """fp16 storage on the fp32 matrix-core kernels (widened exactly on
    load, outputs rounded to nearest even)."""
    compare(2, 2, 333, D, torch.float16, causal, seed=D + 50)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_long_segments_d128(causal, dtype):
    """Two heads over a long ragged sequence at D=128: each segment spans
    many staging rounds and chunks, and the last one ends mid-chunk."""
    m = la()
    assert m.num_segments(1, 2, 20001, 128) < (20001 + 63) // 64
    compare(1, 2, 20001, 128, dtype, causal, seed=11)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_multichunk_segments(causal, dtype):
    """Few heads and a long ragged sequence: segments of several chunks."""
    m = la()
    assert m.num_segments(1, 4, 9000, 64) < (9000 + 63) // 64  # >1 chunk per segment
    compare(1, 4, 9000, 64, dtype, causal, seed=5)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("D", [32, 128])
def test_many_heads_one_segment_each(D, dtype, causal):
    """640 heads, more than the 512 workgroups a launch aims at: every head
    is one segment, and so are the launches sized to the resident
    workgroups.  A ragged N; heads at both ends and in the middle checked."""
    m = la()
    assert m.num_segments(8, 80, 300, D) == 1
    compare(8, 80, 300, D, dtype, causal, heads=[0, 1, 319, 638, 639], seed=D + 7)


# ------------------------------------------------------------- full sizes
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_metric_shape_all_heads(causal, dtype):
    """B=4, H=16, N=4096, D=128, every element of every head."""
    compare(4, 16, 4096, 128, dtype, causal)


@pytest.mark.parametrize("D", [32, 64, 256])
def test_d_sweep(D):
    """D sweep at B=4, H=16, N=4096 fp32 (non-causal); 6 heads checked."""
    compare(4, 16, 4096, D, torch.float32, False, heads=[0, 9, 22, 37, 50, 63])


@pytest.mark.parametrize("N", [1024, 16384, 65536, 131072])
def test_n_sweep_bf16_causal(N):
    """N sweep at B=4, H=16, D=128, bf16 causal; two heads checked at the
    longest lengths, four otherwise."""
    heads = [0, 63] if N >= 65536 else [0, 21, 42, 63]
    compare(4, 16, N, 128, torch.bfloat16, True, heads=heads)


# -------------------------------------------------------------- properties
def test_deterministic():
    say("case deterministic B=2 H=8 N=3000 D=128 causal both")
    q, k, v, g = make_inputs(2, 8, 3000, 128, seed=9, device=DEV)
    for causal in (False, True):
        r1 = run_la(q, k, v, g, causal)
        r2 = run_la(q, k, v, g, causal)
        for a, b in zip(r1, r2):
            assert torch.equal(a, b)


def test_outputs_overwritten_and_guards_intact():
    """NaN-poisoned outputs are fully overwritten; guard words around every
    output stay untouched."""
    m = la()
    B, H, N, D = 1, 3, 333, 64
    say("case guards B=%d H=%d N=%d D=%d" % (B, H, N, D))
    q, k, v, g = make_inputs(B, H, N, D, seed=2, device=DEV)
    n = B * H * N * D
    guard = 256
    for causal in (False, True):
        bufs = [torch.full((n + 2 * guard,), float("nan"), device=DEV) for _ in range(4)]
        views = [b[guard:guard + n].view(B, H, N, D) for b in bufs]
        m.forward(q, k, v, causal, out=views[0])
        m.backward(q, k, v, g, causal, outs=tuple(views[1:]))
        torch.cuda.synchronize()
        for b, vw in zip(bufs, views):
            assert torch.isfinite(vw).all()
            assert torch.isnan(b[:guard]).all() and torch.isnan(b[guard + n:]).all()


def test_heads_independent():
    """Perturbing one head's inputs leaves every other head bit-identical."""
    say("case head isolation B=2 H=3 N=500 D=32")
    q, k, v, g = make_inputs(2, 3, 500, 32, seed=4, device=DEV)
    for causal in (False, True):
        r1 = run_la(q, k, v, g, causal)
        q2, g2 = q.clone(), g.clone()
        q2[1, 2] += 0.5
        g2[1, 2] *= -1
        r2 = run_la(q2, k, v, g2, causal)
        mask = torch.ones(2, 3, dtype=torch.bool)
        mask[1, 2] = False
        for a, b in zip(r1, r2):
            assert torch.equal(a[mask], b[mask])
            assert not torch.equal(a[1, 2], b[1, 2])


@pytest.mark.parametrize("causal", [False, True])
def test_saved_state_equals_recompute(causal):
    m = la()
    say("case state reuse B=2 H=4 N=1500 D=128 causal=%d" % causal)
    q, k, v, g = make_inputs(2, 4, 1500, 128, seed=6, device=DEV)
    _, _, st = m.forward(q, k, v, causal, save_state=True)
    a = m.backward(q, k, v, g, causal, state=st)
    b = m.backward(q, k, v, g, causal, state=None)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_autograd_function():
    m = la()
    say("case autograd B=1 H=2 N=300 D=64")
    q, k, v, g = make_inputs(1, 2, 300, 64, seed=8, device=DEV)
    for causal in (False, True):
        qq, kk, vv = (x.clone().requires_grad_(True) for x in (q, k, v))
        o = m.linear_attention(qq, kk, vv, causal)
        o.backward(g)
        o2, _, _ = m.forward(q, k, v, causal)
        dq, dk, dv = m.backward(q, k, v, g, causal)
        torch.cuda.synchronize()
        assert torch.equal(o.detach(), o2)
        for x, y in zip((qq.grad, kk.grad, vv.grad), (dq, dk, dv)):
            assert torch.equal(x, y)


def test_empty_sequence_is_noop():
    m = la()
    q = torch.zeros(2, 3, 0, 64, device=DEV)
    o, den, _ = m.forward(q, q, q, True, return_den=True)
    dq, dk, dv = m.backward(q, q, q, q, False)
    assert o.shape == q.shape and den.shape == (2, 3, 0) and dq.shape == q.shape


def test_validation_errors_on_device():
    """Bad arguments come back as status codes and launch nothing."""
    m = la()
    q, k, v, g = make_inputs(1, 2, 64, 64, seed=1, device=DEV)
    with pytest.raises(m.LAError) as e:
        m.forward(q, k, v, False, out=q)          # output aliases an input
    assert e.value.code == 6
    big = torch.zeros(2 * 65 * 64, device=DEV)
    strided = big.view(1, 2, 65, 64)[:, :, :64]
    with pytest.raises(ValueError):
        m.forward(strided, k, v)                  # not contiguous
    flat = torch.zeros(2 * 64 * 64 + 1, device=DEV)
    mis = flat[1:].view(1, 2, 64, 64)
    with pytest.raises(m.LAError) as e:
        m.forward(mis, k, v)
    assert e.value.code == 7
    q300 = torch.zeros(1, 2, 64, 300, device=DEV)
    with pytest.raises(m.LAError) as e:
        m.forward(q300, q300, q300)               # head size above 256
    assert e.value.code == 4
    with pytest.raises(m.LAError) as e:
        m.forward(q, k, v, workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    assert e.value.code == 5
    with pytest.raises(TypeError):
        m.forward(q.double(), k.double(), v.double())
    q48 = torch.zeros(1, 2, 64, 48, device=DEV, dtype=torch.float16)
    with pytest.raises(m.LAError) as e:               # a padded size needs the larger workspace
        m.forward(q48, q48, q48, workspace=m.alloc_workspace(1, 2, 64, 32, False, DEV))
    assert e.value.code == 5
