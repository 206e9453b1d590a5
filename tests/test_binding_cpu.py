"""The Python binding checks every caller-supplied buffer before it calls
the library (CPU only: the checks come before the GPU check, so CPU tensors
reach each of them and nothing is launched).  The C side cannot know how big
a buffer is, so an output of the wrong size or type, or a saved state of the
other mask, must be refused here."""
import pytest
import torch

import linear_attention_transformer_amd as la

B, H, N, D = 1, 2, 100, 32


def qkvg(dtype=torch.float32):
    return tuple(torch.zeros(B, H, N, D, dtype=dtype) for _ in range(4))


def test_inputs_valid_but_on_the_cpu_are_refused_last():
    q, k, v, _ = qkvg()
    with pytest.raises(ValueError, match="GPU only"):
        la.forward(q, k, v)


@pytest.mark.parametrize("bad", [torch.zeros(B, H, N, D, dtype=torch.bfloat16),
                                 torch.zeros(B, H, N - 1, D),
                                 torch.zeros(B, H, D, N).transpose(2, 3)])
def test_forward_out_must_match_q(bad):
    q, k, v, _ = qkvg()
    with pytest.raises(ValueError, match="out must be"):
        la.forward(q, k, v, out=bad)


def test_forward_state_out_size_and_type():
    q, k, v, _ = qkvg()
    need = la.state_size(B, H, N, D, True)
    with pytest.raises(ValueError, match="state_out holds"):
        la.forward(q, k, v, True, state_out=torch.zeros(need // 4 - 1))
    with pytest.raises(ValueError, match="state_out must be"):
        la.forward(q, k, v, True, state_out=torch.zeros(need // 8, dtype=torch.float64))


def test_backward_refuses_a_non_causal_state_for_a_causal_call():
    q, k, v, g = qkvg()
    nc = torch.zeros(la.state_size(B, H, N, D, False) // 4)
    assert la.state_size(B, H, N, D, True) > la.state_size(B, H, N, D, False)
    with pytest.raises(ValueError, match="state holds"):
        la.backward(q, k, v, g, True, state=nc)


def test_backward_outs_checked():
    q, k, v, g = qkvg()
    good = torch.zeros_like(q)
    with pytest.raises(ValueError, match="dK must be"):
        la.backward(q, k, v, g, outs=(good, torch.zeros(B, H, N, D + 1), good))
    with pytest.raises(ValueError, match="outs"):
        la.backward(q, k, v, g, outs=(good, good))
    with pytest.raises(ValueError, match="outs"):
        la.backward(q, k, v, g, outs=(good, None, good))


def test_segment_calls_check_their_buffers():
    q, k, v, g = qkvg()
    with pytest.raises(ValueError, match="carry_in"):
        la.forward_segment(q, k, v, carry_in=torch.zeros(B, H, D * D))
    with pytest.raises(ValueError, match="state_out holds"):
        la.forward_segment(q, k, v, True, state_out=torch.zeros(4))
    with pytest.raises(ValueError, match="out must be"):
        la.forward_segment(q, k, v, out=torch.zeros(1))
    with pytest.raises(ValueError, match="outs must be"):
        la.backward_segment(q, k, v, g, outs=(torch.zeros_like(q), torch.zeros_like(q), None))
    with pytest.raises(ValueError, match="state holds"):
        la.backward_segment(q, k, v, g, True, state=torch.zeros(4))


def test_decode_step_out_checked():
    q = torch.zeros(B, H, D)
    with pytest.raises(ValueError, match="out must be"):
        la.decode_step(q, q, q, out=torch.zeros(B, H, D, dtype=torch.float16))


def test_layer_buffers_checked():
    Bn, Nn, C, Hh, Dd = 1, 16, 32, 2, 8
    x = torch.zeros(Bn, Nn, C)
    wqkv = torch.zeros(C, 3 * Hh * Dd)
    wo = torch.zeros(Hh * Dd, C)
    sb, _ = la.layer_sizes(Bn, Nn, C, Hh, Dd)
    with pytest.raises(ValueError, match="saved holds"):
        la.layer_forward(x, wqkv, wo, Hh, saved=torch.zeros(sb - 1, dtype=torch.uint8))
    with pytest.raises(ValueError, match="saved buffer"):
        la.layer_backward(x, wqkv, wo, x, Hh, saved=None)
    with pytest.raises(ValueError, match="dWo must be"):
        la.layer_backward(x, wqkv, wo, x, Hh, saved=torch.zeros(sb, dtype=torch.uint8),
                          outs=(torch.zeros_like(x), torch.zeros_like(wqkv), torch.zeros(3)))
