"""GPU parity of the carried-state calls (la_forward_segment /
la_backward_segment) against the fp64 oracle (marked gpu).

The carried records are formed by the oracle from seeded tokens outside the
piece (so their magnitudes are those of real prefixes and suffixes), rounded
to fp32, and given to both sides.  O, den, dQ, dK, dV and the outgoing
records are compared element by element at the same tolerances as the plain
calls (fp32 storage 1e-5, bf16 storage 2e-2, fp16 storage 1e-3): tensor-wide,
head by head and row by row (tests/parity_checks.py; a record's rows are the
D rows of its matrix and its two vectors).
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


def f64(t):
    return t.detach().double().cpu().numpy()


def carries(B, H, D, dtype, causal, n_before, n_after, seed):
    """fp32 carry records from seeded tokens around a piece: the forward
    record of n_before tokens and the gradient record of n_after rows."""
    qa, ka, va, ga = make_inputs(B, H, n_before + n_after, D, dtype=dtype, seed=seed + 1000)
    a = [as_f64_numpy(x) for x in (qa, ka, va, ga)]
    pre = [x[:, :, :n_before] for x in a]
    post = [x[:, :, n_before:] for x in a]
    _, _, rec = oracle.forward_carry(pre[0], pre[1], pre[2], causal)
    *_, grec = oracle.backward_carry(post[0], post[1], post[2], post[3], causal,
                                     rec, n_before)
    t = lambda r: torch.from_numpy(r).float().to(DEV)  # noqa: E731
    return t(rec), t(grec)


def check(name, got, ref, D, heads, errs, tol):
    """Append the error measures of one output (den: per element, against
    its own value; everything else: rows of D values)."""
    x = f64(got).reshape(ref.shape)
    assert np.all(np.isfinite(x)), name
    den = name.startswith("den")
    errs.append((name, pc.metrics(x, ref, 1 if den else D, heads,
                                  floor=0.0 if den else pc.row_floor(tol))))


@pytest.mark.parametrize("D", [6, 16, 32, 64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_segment_parity(D, causal, dtype):
    """One ragged piece (N=300, five segments) with both carries, every head
    size (each kernel family), both masks and storage types."""
    m = la()
    B, H, N, nb, na = 1, 2, 300, 123, 77
    say("case segment B=%d H=%d N=%d D=%d %s causal=%d carry=%d/%d"
        % (B, H, N, D, dtype, causal, nb, na))
    q, k, v, g = make_inputs(B, H, N, D, dtype=dtype, seed=D + 7, device=DEV)
    cin, gin = carries(B, H, D, dtype, causal, nb, na, seed=D)
    o, den, cout, st = m.forward_segment(q, k, v, causal, carry_in=cin, n_carry=nb,
                                         return_den=True, save_state=True)
    dq, dk, dv, gout = m.backward_segment(q, k, v, g, causal, carry_in=cin, n_carry=nb,
                                          gcarry_in=gin, state=st)
    # the same backward with the state recomputed from carry_in
    dq2, dk2, dv2, gout2 = m.backward_segment(q, k, v, g, causal, carry_in=cin, n_carry=nb,
                                              gcarry_in=gin)
    torch.cuda.synchronize()
    a = [as_f64_numpy(x) for x in (q, k, v, g)]
    rin, grin = f64(cin), f64(gin)
    o_r, den_r, cout_r = oracle.forward_carry(a[0], a[1], a[2], causal, rin, nb)
    dq_r, dk_r, dv_r, gout_r = oracle.backward_carry(*a, causal, rin, nb, grin)
    errs = []
    for name, x, r in (("O", o, o_r), ("den", den, den_r), ("carry_out", cout, cout_r),
                       ("dQ", dq, dq_r), ("dK", dk, dk_r), ("dV", dv, dv_r),
                       ("gcarry_out", gout, gout_r)):
        check(name, x, r, D, B * H, errs, TOL[dtype])
    pc.check_all(errs, TOL[dtype], say)
    for x, y in ((dq, dq2), (dk, dk2), (dv, dv2), (gout, gout2)):
        assert torch.equal(x, y)


def _pieces(N, cuts):
    out, s = [], 0
    for c in cuts + [N]:
        out.append(slice(s, c))
        s = c
    return out


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_pieces_equal_whole_sequence(causal, dtype):
    """A 5000-token sequence at D=128 cut into three ragged pieces gives the
    whole-sequence outputs of la_forward / la_backward.  Causal: a stream
    (forward in order, backward in reverse).  Non-causal: the sharded use,
    each piece's own records first (no outputs), then the full calls with
    the sum of the other pieces' records."""
    m = la()
    B, H, N, D = 1, 4, 5000, 128
    say("case pieces B=%d H=%d N=%d D=%d %s causal=%d" % (B, H, N, D, dtype, causal))
    q, k, v, g = make_inputs(B, H, N, D, dtype=dtype, seed=5, device=DEV)
    o_w, den_w, _ = m.forward(q, k, v, causal, return_den=True)
    dq_w, dk_w, dv_w = m.backward(q, k, v, g, causal)
    cuts = _pieces(N, [1100, 3600])
    P = lambda x, c: x[:, :, c].contiguous()  # noqa: E731
    outs = {}
    if causal:
        rec, n0, fwd = None, 0, []
        for c in cuts:
            o, den, rec_next, st = m.forward_segment(P(q, c), P(k, c), P(v, c), True,
                                                     carry_in=rec, n_carry=n0,
                                                     return_den=True, save_state=True)
            fwd.append((rec, n0, st))
            outs[c.start] = [o, den]
            rec, n0 = rec_next, n0 + (c.stop - c.start)
        grec = None
        for c, (rec, n0, st) in reversed(list(zip(cuts, fwd))):
            dq, dk, dv, grec = m.backward_segment(P(q, c), P(k, c), P(v, c), P(g, c), True,
                                                  carry_in=rec, n_carry=n0, gcarry_in=grec,
                                                  state=st)
            outs[c.start] += [dq, dk, dv]
    else:
        own = [m.forward_segment(P(q, c), P(k, c), P(v, c), False, compute_out=False)[2]
               for c in cuts]
        tot = sum(own[1:], own[0].clone())
        fr = []
        for i, c in enumerate(cuts):
            others = sum((r for j, r in enumerate(own) if j != i), torch.zeros_like(own[0]))
            n0 = N - (c.stop - c.start)
            o, den, cout, _ = m.forward_segment(P(q, c), P(k, c), P(v, c), False,
                                                carry_in=others, n_carry=n0, return_den=True)
            torch.testing.assert_close(cout, tot, rtol=1e-5, atol=1e-4)
            fr.append((others, n0))
            outs[c.start] = [o, den]
        gown = []
        for c, (others, n0) in zip(cuts, fr):
            _, dk, dv, gr = m.backward_segment(P(q, c), P(k, c), P(v, c), P(g, c), False,
                                               carry_in=others, n_carry=n0, compute_kv=False)
            assert dk is None and dv is None
            gown.append(gr)
        for i, (c, (others, n0)) in enumerate(zip(cuts, fr)):
            gothers = sum((r for j, r in enumerate(gown) if j != i), torch.zeros_like(gown[0]))
            dq, dk, dv, _ = m.backward_segment(P(q, c), P(k, c), P(v, c), P(g, c), False,
                                               carry_in=others, n_carry=n0, gcarry_in=gothers)
            outs[c.start] += [dq, dk, dv]
    torch.cuda.synchronize()
    whole = (o_w, den_w, dq_w, dk_w, dv_w)
    errs = []
    for i, name in enumerate(("O", "den", "dQ", "dK", "dV")):
        got = torch.cat([outs[c.start][i] for c in cuts], dim=2)
        check(name, got, f64(whole[i]), D, B * H, errs, TOL[dtype])
    say("  against the whole sequence:")
    pc.check_all(errs, TOL[dtype], say)


def test_zero_length_piece_passes_records_through():
    m = la()
    B, H, D = 2, 3, 64
    say("case zero-length piece B=%d H=%d D=%d" % (B, H, D))
    e = torch.empty(B, H, 0, D, device=DEV)
    cin, gin = carries(B, H, D, torch.float32, True, 50, 20, seed=1)
    _, _, cout, _ = m.forward_segment(e, e, e, True, carry_in=cin, n_carry=50)
    _, _, _, gout = m.backward_segment(e, e, e, e, True, carry_in=cin, n_carry=50,
                                       gcarry_in=gin)
    _, _, zout, _ = m.forward_segment(e, e, e, False)
    torch.cuda.synchronize()
    assert torch.equal(cout, cin) and torch.equal(gout, gin)
    assert torch.count_nonzero(zout).item() == 0


def test_large_carried_count_and_state_only_call():
    """A count of 2^30 carried tokens with a zero record (only the constant
    term of those tokens), and the records-only forward matching the full
    call's carry_out bit for bit."""
    m = la()
    B, H, N, D = 1, 2, 500, 64
    say("case large carried count B=%d H=%d N=%d D=%d" % (B, H, N, D))
    q, k, v, g = make_inputs(B, H, N, D, dtype=torch.float32, seed=9, device=DEV)
    n0 = 1 << 30
    o, den, cout, _ = m.forward_segment(q, k, v, False, n_carry=n0, return_den=True)
    _, _, cout2, _ = m.forward_segment(q, k, v, False, compute_out=False)
    torch.cuda.synchronize()
    a = [as_f64_numpy(x) for x in (q, k, v)]
    o_r, den_r, _ = oracle.forward_carry(*a, False, None, n0)
    assert rel_l2(f64(o), o_r) <= 1e-5 and rel_l2(f64(den), den_r) <= 1e-6
    assert torch.equal(cout, cout2)


# ------------------------------------------------------------ decode step
@pytest.mark.parametrize("D", [6, 16, 32, 64, 100, 128, 256])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_decode_step_parity(D, dtype):
    """One decode step for B=3 sequences of different lengths (per-sequence
    counts on the device) against the oracle's one-token causal piece."""
    m = la()
    B, H = 3, 2
    lens = [0, 37, 190]
    say("case decode B=%d H=%d D=%d %s prefixes=%s" % (B, H, D, dtype, lens))
    q, k, v, _ = make_inputs(B, H, 1, D, dtype=dtype, seed=D + 3, device=DEV)
    recs = []
    for b, n in enumerate(lens):
        qa, ka, va, _ = make_inputs(1, H, max(n, 1), D, dtype=dtype, seed=100 + b)
        a = [as_f64_numpy(x)[:, :, :n] for x in (qa, ka, va)]
        recs.append(oracle.forward_carry(*a, True)[2])
    rin = torch.from_numpy(np.concatenate(recs, axis=0)).float().to(DEV)
    counts = torch.tensor(lens, dtype=torch.int64, device=DEV)
    o, den, rout = m.decode_step(q[:, :, 0].contiguous(), k[:, :, 0].contiguous(),
                                 v[:, :, 0].contiguous(), rin, counts=counts, return_den=True)
    torch.cuda.synchronize()
    a = [as_f64_numpy(x) for x in (q, k, v)]
    r64 = f64(rin)
    errs = []
    for b, n in enumerate(lens):
        sb = slice(b, b + 1)
        o_r, den_r, rec_r = oracle.forward_carry(a[0][sb], a[1][sb], a[2][sb], True, r64[sb], n)
        check("O[%d]" % b, o[sb], o_r, D, H, errs, TOL[dtype])
        check("den[%d]" % b, den[sb], den_r, D, H, errs, TOL[dtype])
        check("state_out[%d]" % b, rout[sb], rec_r, D, H, errs, TOL[dtype])
    pc.check_all(errs, TOL[dtype], say)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("prefill", [0, 300])
def test_decode_chain_equals_causal_forward(dtype, prefill):
    """A prefill through la_forward_segment (or none), then 40 decode steps
    alternating two state buffers, gives the rows of one causal la_forward
    over the whole sequence (B=2 H=8 D=128)."""
    m = la()
    B, H, D, T = 2, 8, 128, 40
    N = prefill + T
    say("case decode chain B=%d H=%d D=%d %s prefill=%d steps=%d" % (B, H, D, dtype, prefill, T))
    q, k, v, _ = make_inputs(B, H, N, D, dtype=dtype, seed=21, device=DEV)
    o_w, den_w, _ = m.forward(q, k, v, True, return_den=True)
    bufs = [m.new_record(B, H, D, DEV), m.new_record(B, H, D, DEV)]
    state = None
    if prefill:
        P = lambda x: x[:, :, :prefill].contiguous()  # noqa: E731
        m.forward_segment(P(q), P(k), P(v), True, carry_out=bufs[0], compute_out=False)
        state = bufs[0]
    outs, dens = [], []
    for t in range(T):
        i = prefill + t
        tok = lambda x: x[:, :, i].contiguous()  # noqa: E731
        nxt = bufs[(t + 1) % 2] if prefill else bufs[t % 2]
        o, den, state = m.decode_step(tok(q), tok(k), tok(v), state, state_out=nxt,
                                      n_prev=i, return_den=True)
        outs.append(o)
        dens.append(den)
    torch.cuda.synchronize()
    got_o = torch.stack(outs, dim=2)
    got_d = torch.stack(dens, dim=2)
    eo = rel_l2(f64(got_o), f64(o_w[:, :, prefill:]))
    ed = rel_l2(f64(got_d), f64(den_w[:, :, prefill:]))
    say("  rel-L2 vs whole O=%.2e den=%.2e" % (eo, ed))
    assert eo <= TOL[dtype] and ed <= 1e-5


def test_decode_steps_replayed_from_a_graph():
    """Six decode steps captured in a HIP graph (the call allocates nothing
    and issues no memset) replay to the eager results, three times, with
    eager work and synchronisation between the replays."""
    m = la()
    B, H, D, T = 2, 4, 64, 6
    say("case decode graph B=%d H=%d D=%d steps=%d" % (B, H, D, T))
    q, k, v, _ = make_inputs(B, H, T, D, dtype=torch.float32, seed=4, device=DEV)
    toks = [[x[:, :, t].contiguous() for x in (q, k, v)] for t in range(T)]
    start = torch.randn(B, H, D * D + 2 * D, device=DEV).abs_() * 0.01
    recs = [m.new_record(B, H, D, DEV), m.new_record(B, H, D, DEV)]
    outs = [torch.empty(B, H, D, device=DEV) for _ in range(T)]

    def run():
        for t in range(T):
            m.decode_step(*toks[t], recs[t % 2], state_out=recs[(t + 1) % 2], n_prev=50 + t,
                          out=outs[t])

    recs[0].copy_(start)
    run()
    torch.cuda.synchronize()
    ref_o = [x.clone() for x in outs]
    ref_s = recs[T % 2].clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        recs[0].copy_(start)
        run()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        for x in outs:
            x.zero_()
        recs[0].copy_(start)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t in range(T):
            assert torch.equal(outs[t], ref_o[t]), (rep, t)
        assert torch.equal(recs[T % 2], ref_s), rep
