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

from tests import parity_checks as pc

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


def den_report(den_ref, N, causal, gate=True):
    """min and max of den_i / count_i (count_i = rows each row sees).  The
    inputs must keep every denominator well away from zero (no guard in the
    method: a row whose den is near 0 is ill-conditioned).  With the input
    recipe q.k has variance 1/D, so below D = 16 the first causal rows can
    reach den <= 0; those cases only report it (gate=False)."""
    cnt = np.arange(1, N + 1, dtype=np.float64) if causal else np.full(N, float(N))
    ratio = den_ref.reshape(-1, N) / cnt
    lo, hi = float(ratio.min()), float(ratio.max())
    say("  den/count min %.3f max %.3f%s" % (lo, hi, "" if gate else " (report only)"))
    if gate:
        assert lo > 0.1, "inputs give an ill-conditioned denominator (den/count %.3f)" % lo
    return lo, hi


def compare(B, H, N, D, dtype, causal, heads=None, seed=0, lin_gate=True, inputs=None):
    """Run the HIP path on the full problem; check `heads` (all if None)
    tensor-wide, head by head and row by row (tests/parity_checks.py)."""
    say("case B=%d H=%d N=%d D=%d %s causal=%d seed=%d" % (B, H, N, D, dtype, causal, seed))
    if inputs is None:
        q, k, v, g = make_inputs(B, H, N, D, dtype=dtype, seed=seed, device=DEV)
    else:
        q, k, v, g = inputs
    got = run_la(q, k, v, g, causal)
    if heads is None:
        sel = lambda t: t
        nh = B * H
    else:
        idx = torch.tensor(heads, device=DEV)
        sel = lambda t: t.reshape(B * H, *t.shape[2:]).index_select(0, idx).unsqueeze(0)
        nh = len(heads)
    a = [as_f64_numpy(sel(x)) for x in (q, k, v, g)]
    o_ref, den_ref = oracle.forward_state(a[0], a[1], a[2], causal)
    refs = (o_ref, den_ref) + tuple(oracle.backward_state(*a, causal))
    tol = TOL[dtype]
    if N > 0:
        den_report(den_ref, N, causal, gate=D >= 16)
    # dQ and dK vanish in exact arithmetic when every row sees one token
    # (N = 1); their error is then measured against the gradient scale of
    # the same loss, ||dV|| (never zero: its rows sum to those of dO).
    gscale = float(np.linalg.norm(refs[4]))
    results = []
    for name, x, r in zip(("O", "den", "dQ", "dK", "dV"), got, refs):
        xs = as_f64_numpy(sel(x)).reshape(r.shape)
        assert np.all(np.isfinite(xs)), name
        sc = gscale if name in ("dQ", "dK") and N == 1 else 0.0
        width = 1 if name == "den" else D
        fl = 0.0 if name == "den" else pc.row_floor(tol)
        results.append((name, pc.metrics(xs, r, width, nh, floor=fl, scale=sc)))
    pc.check_all(results, tol, say)
    if lin_gate and N > 1:
        # the linear term alone: O - O(Q=0) against the oracle's; gated for
        # fp32, reported for 16-bit storage (whose output rounding alone is
        # a few per cent of this small part of O)
        o0_ref, _ = oracle.forward_state(0 * a[0], a[1], a[2], causal)
        lin = as_f64_numpy(sel(got[0])).reshape(o_ref.shape) - o0_ref
        e = rel_l2(lin, o_ref - o0_ref)
        say("  linear-term rel-L2 %.2e%s" % (e, "" if dtype == torch.float32 else " (report only)"))
        if dtype == torch.float32:
            assert e <= 1e-4
    return got


# ------------------------------------------------------------ small sizes
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_tiny_head(causal, dtype):
    """B=1, H=2, N=64, D=16 (the tiny workload)."""
    compare(1, 2, 64, 16, dtype, causal)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_figure1_shape(causal, dtype):
    """B=2, H=4, N=8, D=6: the shape the Figure 1 caption of the
    sciencestack.ai page draws (its reduction block L=2 is a tuning choice
    here)."""
    compare(2, 4, 8, 6, dtype, causal, seed=1)


@pytest.mark.parametrize("N", [63, 65, 4097])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_lengths_around_chunks(N, causal, dtype):
    """One row short of, one past, a 64-row chunk and a 4096-row sequence,
    at D = 128."""
    compare(1, 4, N, 128, dtype, causal, seed=N)


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
    """Head sizes between the native ones (D = 6 is the Figure 1 shape):
    D <= 16 at width 16 on the caller's rows, the others padded to the next
    native size inside the library."""
    compare(2, 2, 333, D, dtype, causal, seed=D + 40)


@pytest.mark.parametrize("D", [1, 6, 16])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_narrow_heads_without_padded_copies(D, causal, dtype):
    """Heads of D <= 16 run at width 16 on the caller's own rows: the
    forward and the backward launch no stage / unstage pass, and both match
    the oracle.  (The seeds of test_generic_head_sizes: below D = 16 the
    recipe's q.k can bring a causal denominator near zero, and these inputs
    keep every den/count well above it.)"""
    q, k, v, g = make_inputs(2, 2, 333, D, dtype=dtype, seed=D + 40, device=DEV)
    m = la()
    tf, tb = m.KernelTrace(DEV), m.KernelTrace(DEV)
    _, _, st = m.forward(q, k, v, causal, save_state=True, trace=tf)
    m.backward(q, k, v, g, causal, state=st, trace=tb)
    torch.cuda.synchronize()
    names = tf.names() + tb.names()
    say("  launches: " + " ".join(names))
    assert names and not [n for n in names if n in ("stage", "unstage")], names
    compare(2, 2, 333, D, dtype, causal, seed=D + 40, inputs=(q, k, v, g))


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


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_causal_d256_full_size(dtype):
    """B=4, H=16, N=4096, D=256 causal: the eight-wave chunk walks over
    512-row segments (a 256 x 32 state slab per wave); heads at both ends and
    in the middle, head by head and row by row."""
    compare(4, 16, 4096, 256, dtype, True, heads=[0, 1, 31, 62, 63], seed=9)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_causal_merged_walk_odd_segments(dtype):
    """B=4, H=16, N=640, D=128 causal: five 128-row segments per head, more
    workgroups than one batch of the one-workgroup dK | dV walk holds, so its
    workgroups walk two segments each and the last one walks a single
    segment; every head, head by head and row by row."""
    assert la().num_segments(4, 16, 640, 128) == 5
    compare(4, 16, 640, 128, dtype, True, seed=11)


@pytest.mark.parametrize("D", [32, 64, 256])
def test_d_sweep(D):
    """D sweep at B=4, H=16, N=4096 fp32 (non-causal); every head checked,
    head by head and row by row."""
    compare(4, 16, 4096, D, torch.float32, False)


@pytest.mark.parametrize("N", [1024, 16384, 65536, 131072])
def test_n_sweep_bf16_causal(N):
    """N sweep at B=4, H=16, D=128, bf16 causal: every head at N = 1024,
    sixteen heads spread over the batch (both ends included) at the longer
    lengths; each checked head by head and row by row."""
    heads = None if N <= 4096 else list(range(0, 64, 4)) + [63]
    compare(4, 16, N, 128, torch.bfloat16, True, heads=heads)


# ------------------------------------------------------- closed forms on the GPU
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_constant_v_gives_constant_o(causal, dtype):
    """Every value row equal to one vector v: each output row is v, since the
    weights of a row sum to its denominator.  bf16 storage: the fp32 result
    is within far less than half a bf16 step of the stored v, so it rounds
    back to v bit for bit.  Also: the columns of dV sum to those of dO."""
    B, H, N, D = 2, 4, 1000, 128
    say("case constant V B=%d H=%d N=%d D=%d %s causal=%d" % (B, H, N, D, dtype, causal))
    q, k, v, g = make_inputs(B, H, N, D, dtype=dtype, seed=21, device=DEV)
    v = v[:, :, :1].expand(B, H, N, D).contiguous()
    o, den, dq, dk, dv = run_la(q, k, v, g, causal)
    if dtype == torch.bfloat16:
        assert torch.equal(o, v)
    else:
        m = pc.metrics(as_f64_numpy(o), as_f64_numpy(v), D, B * H,
                       floor=pc.row_floor(TOL[dtype]))
        pc.check_all([("O", m)], TOL[dtype], say)
    sdv = as_f64_numpy(dv).sum(axis=2)
    sdo = as_f64_numpy(g).sum(axis=2)
    e = rel_l2(sdv, sdo)
    say("  sum dV vs sum dO rel %.2e" % e)
    assert e <= TOL[dtype]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_zero_q_gives_running_mean(causal, dtype):
    """Q = 0: every weight is 1, so den_i is the count of rows seen (exactly),
    o_i is the mean (running mean when causal) of the value rows it sees,
    and dK = Q-weighted sums vanish exactly."""
    B, H, N, D = 2, 3, 777, 64
    say("case Q=0 B=%d H=%d N=%d D=%d %s causal=%d" % (B, H, N, D, dtype, causal))
    q, k, v, g = make_inputs(B, H, N, D, dtype=dtype, seed=22, device=DEV)
    q = torch.zeros_like(q)
    o, den, dq, dk, dv = run_la(q, k, v, g, causal)
    vv = as_f64_numpy(v)
    if causal:
        cnt = np.arange(1, N + 1, dtype=np.float64)
        mean = np.cumsum(vv, axis=2) / cnt[:, None]
    else:
        cnt = np.full(N, float(N))
        mean = np.broadcast_to(vv.mean(axis=2, keepdims=True), vv.shape)
    assert np.array_equal(as_f64_numpy(den), np.broadcast_to(cnt, (B, H, N)))
    assert int(torch.count_nonzero(dk)) == 0
    m = pc.metrics(as_f64_numpy(o), mean, D, B * H, floor=pc.row_floor(TOL[dtype]))
    pc.check_all([("O", m)], TOL[dtype], say)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_wider_denominators(causal, dtype):
    """Q and K scaled up (x4 non-causal, x2 causal) so that q.k is no longer
    small against the constant term and den_i / count_i spreads (reported;
    the causal scale keeps its minimum above 0.1)."""
    B, H, N, D = 2, 8, 2000, 128
    s = 2.0 if causal else 4.0
    q, k, v, g = make_inputs(B, H, N, D, dtype=torch.float32, seed=23, device=DEV)
    ins = tuple(x.to(dtype) for x in (q * s, k * s, v, g))
    compare(B, H, N, D, dtype, causal, seed=23, inputs=ins)


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


def test_pending_hip_error_is_left_to_its_owner():
    """An error that an earlier HIP call on this thread left pending (here a
    hipSetDevice to a device that does not exist: a host-side refusal that
    reaches no GPU) is not reported as the library's own: la_forward
    launches nothing, returns LA_ERR_HIP_PENDING and leaves the error
    pending for its owner; the next call runs normally."""
    import ctypes
    m = la()
    lib = m.load_library()
    hip = ctypes.CDLL("libamdhip64.so")
    B, H, N, D = 1, 2, 64, 64
    say("case pending HIP error B=%d H=%d N=%d D=%d" % (B, H, N, D))
    q, k, v, _ = make_inputs(B, H, N, D, seed=1, device=DEV)
    out = torch.full_like(q, 3.0)
    ws = m.alloc_workspace(B, H, N, D, False, DEV)
    torch.cuda.synchronize()
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    args = (P(q), P(k), P(v), P(out), B, H, N, D, 0, m.LA_FP32, None, None, P(ws),
            ws.numel(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    hip.hipGetLastError()                           # start from a clear state
    bad = hip.hipSetDevice(9999)
    assert bad != 0
    if hip.hipPeekAtLastError() != bad:
        hip.hipGetLastError()
        pytest.skip("this HIP runtime does not keep the refused call's error pending")
    rc = lib.la_forward(*args)
    assert rc == 9, m.status_string(rc)
    assert hip.hipGetLastError() == bad             # still pending; now cleared
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())                 # nothing was launched
    assert lib.la_forward(*args) == 0
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()) and not bool((out == 3.0).all())
