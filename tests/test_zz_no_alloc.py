"""la_forward_noalloc (the forward on the library's static device workspace,
for callers that cannot allocate) against la_forward (marked gpu).

Two calls in a row on one device share the static array: the second, with a
smaller input, must not see anything of the first.  Both are compared with
la_forward on the same inputs (the same kernels and launch plan, so bit for
bit) and with the fp64 oracle at the storage type's tolerance.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from linear_attention_transformer_amd.inputs import as_f64_numpy, make_inputs
from tests import parity_checks as pc

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2, torch.float16: 1e-3}


def la():
    import linear_attention_transformer_amd as m
    m.load_library()
    return m


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def one_call(m, B, H, N, D, dtype, causal, seed):
    say("case no-alloc forward B=%d H=%d N=%d D=%d %s causal=%d" % (B, H, N, D, dtype, causal))
    q, k, v, _ = make_inputs(B, H, N, D, dtype=dtype, seed=seed, device=DEV)
    out = torch.full_like(q, float("nan"))
    den = torch.full((B, H, N), float("nan"), device=DEV)
    st = torch.empty(max(m.state_size(B, H, N, D, causal) // 4, 4), device=DEV)
    m.forward_noalloc(q, k, v, causal, out=out, den_out=den, state_out=st)
    o_ref, den_ref, st_ref = m.forward(q, k, v, causal, return_den=True, save_state=True)
    torch.cuda.synchronize()
    return (q, k, v), (out, den, st), (o_ref, den_ref, st_ref)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_noalloc_forward_matches_la_forward(dtype, causal):
    m = la()
    first = (4, 16, 4096, 128)          # the workload shape: 38 MB of workspace
    second = (1, 3, 777, 64)            # smaller, ragged, after it
    for (B, H, N, D), seed in ((first, 3), (second, 4)):
        ins, got, ref = one_call(m, B, H, N, D, dtype, causal, seed)
        for name, x, y in zip(("O", "den", "state"), got, ref):
            assert torch.equal(x, y), name
        a = [as_f64_numpy(t) for t in ins]
        o_r, den_r = oracle.forward_state(*a, causal)
        res = [("O", pc.metrics(as_f64_numpy(got[0]), o_r, D, B * H,
                                floor=pc.row_floor(TOL[dtype]))),
               ("den", pc.metrics(as_f64_numpy(got[1]), den_r, 1, B * H, floor=0.0))]
        pc.check_all(res, TOL[dtype], say)


def test_noalloc_forward_padded_head_size_and_limit():
    """A padded head size (D = 20) within the static workspace, and a call
    whose workspace would exceed it (D = 256 at B4 H16 N4096: 152 MB)
    refused before any launch."""
    m = la()
    ins, got, ref = one_call(m, 2, 2, 300, 20, torch.float32, True, 5)
    for x, y in zip(got[:2], ref[:2]):
        assert torch.equal(x, y)
    q = torch.zeros(4, 16, 4096, 256, device=DEV)
    out = torch.full_like(q, 7.0)
    with pytest.raises(m.LAError) as e:
        m.forward_noalloc(q, q, q, False, out=out)
    assert e.value.code == 5
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


def test_noalloc_forward_in_a_captured_graph():
    """Captured in a HIP graph (no allocation, no memset node) and replayed
    three times, with eager work between the replays: each replay equals
    la_forward."""
    m = la()
    B, H, N, D = 2, 8, 1500, 128
    say("case no-alloc forward graph B=%d H=%d N=%d D=%d" % (B, H, N, D))
    q, k, v, _ = make_inputs(B, H, N, D, seed=6, device=DEV)
    out = torch.empty_like(q)
    ref, _, _ = m.forward(q, k, v, True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        m.forward_noalloc(q, k, v, True, out=out)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        m.forward_noalloc(q, k, v, True, out=out)
    for _ in range(3):
        out.fill_(float("nan"))
        m.forward(q, k, v, False)          # other work on the same device between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
