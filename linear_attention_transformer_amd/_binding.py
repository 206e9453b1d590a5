"""ctypes binding of liblinattn.so (C ABI in include/la.h).

Argument marshalling only: every step of the forward and backward pass runs
in the HIP kernels of the library.  PyTorch provides device memory and the
current stream.  There is no CPU fallback: if the library is missing or a
tensor is not on the GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblinattn.so")

LA_FP32, LA_BF16, LA_FP16 = 0, 1, 2
STATUS = {0: "LA_OK", 1: "LA_ERR_NULL", 2: "LA_ERR_SHAPE", 3: "LA_ERR_DTYPE",
          4: "LA_ERR_UNSUPPORTED", 5: "LA_ERR_WORKSPACE", 6: "LA_ERR_ALIAS",
          7: "LA_ERR_ALIGN", 8: "LA_ERR_HIP", 9: "LA_ERR_HIP_PENDING"}
SUPPORTED_D = tuple(range(1, 257))      # every head size the library takes
NATIVE_D = (32, 64, 128, 256)            # run at their own width
NARROW_D = tuple(range(1, 17))           # run at width 16 on the caller's rows (no padded copies)

_lib = None


class LAError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__("%s failed: %s" % (what, status_string(code)))


def load_library():
    """Load liblinattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "HIP library %s is not built; run __graft_entry__.build() "
            "(or python -m linear_attention_transformer_amd.build)" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, sz, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.la_status_string.argtypes = [ci]
    lib.la_status_string.restype = ctypes.c_char_p
    lib.la_workspace_size.argtypes = [i64, i64, i64, i64, ci]
    lib.la_workspace_size.restype = sz
    lib.la_workspace_size_for.argtypes = [i64, i64, i64, i64, ci, ci]
    lib.la_workspace_size_for.restype = sz
    lib.la_state_size.argtypes = [i64, i64, i64, i64, ci]
    lib.la_state_size.restype = sz
    lib.la_num_segments.argtypes = [i64, i64, i64, i64, ci]
    lib.la_num_segments.restype = i64
    lib.la_forward.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, ci, ci, vp, vp,
                               vp, sz, vp]
    lib.la_forward.restype = ci
    lib.la_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, ci,
                                ci, vp, vp, sz, vp]
    lib.la_backward.restype = ci
    lib.la_record_size.argtypes = [i64, i64, i64]
    lib.la_record_size.restype = sz
    lib.la_forward_segment.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, ci, ci, vp, i64,
                                       vp, vp, vp, vp, sz, vp]
    lib.la_forward_segment.restype = ci
    lib.la_backward_segment.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, ci,
                                        ci, vp, i64, vp, vp, vp, vp, sz, vp]
    lib.la_backward_segment.restype = ci
    lib.la_layer_saved_size.argtypes = [i64, i64, i64, i64, i64, ci, ci]
    lib.la_layer_saved_size.restype = sz
    lib.la_layer_workspace_size.argtypes = [i64, i64, i64, i64, i64, ci, ci]
    lib.la_layer_workspace_size.restype = sz
    lib.la_layer_forward.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, ci, ci, vp, vp,
                                     sz, vp]
    lib.la_layer_forward.restype = ci
    lib.la_layer_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ci,
                                      ci, vp, vp, sz, vp]
    lib.la_layer_backward.restype = ci
    lib.la_decode_step.argtypes = [vp, vp, vp, vp, i64, i64, i64, ci, vp, vp, vp, i64, vp, vp]
    lib.la_decode_step.restype = ci
    lib.la_forward_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, ci, ci, vp, vp, vp]
    lib.la_forward_noalloc.restype = ci
    ev, ip, cpp = ctypes.c_void_p, ctypes.POINTER(ci), ctypes.POINTER(ctypes.c_char_p)
    lib.la_forward_traced.argtypes = lib.la_forward.argtypes + [ev, ci, ip, cpp]
    lib.la_forward_traced.restype = ci
    lib.la_backward_traced.argtypes = lib.la_backward.argtypes + [ev, ci, ip, cpp]
    lib.la_backward_traced.restype = ci
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load_library().la_status_string(int(code)).decode()


def workspace_size(B, H, N, D, causal=False, dtype=None) -> int:
    """Workspace bytes; `dtype` (a torch dtype) matters for fp16 storage."""
    if dtype is None:
        return int(load_library().la_workspace_size(B, H, N, D, int(bool(causal))))
    return int(load_library().la_workspace_size_for(B, H, N, D, int(bool(causal)),
                                                    _dtype_of(dtype)))


def state_size(B, H, N, D, causal=False) -> int:
    return int(load_library().la_state_size(B, H, N, D, int(bool(causal))))


def num_segments(B, H, N, D, causal=False) -> int:
    return int(load_library().la_num_segments(B, H, N, D, int(bool(causal))))


def record_size(B, H, D) -> int:
    return int(load_library().la_record_size(B, H, D))


def _dtype_of(dt) -> int:
    if dt == torch.float32:
        return LA_FP32
    if dt == torch.bfloat16:
        return LA_BF16
    if dt == torch.float16:
        return LA_FP16
    raise TypeError("linear attention supports float32, bfloat16 and float16 storage, got %s"
                    % dt)


def _dtype_code(t: torch.Tensor) -> int:
    return _dtype_of(t.dtype)


def _check(*ts: torch.Tensor):
    """Inputs q, k, v (and dO): one shape [B, H, N, D], dtype and device,
    contiguous.  (The GPU check comes last, in _on_gpu, after every buffer
    has been checked.)"""
    t0 = ts[0]
    if t0.dim() != 4:
        raise ValueError("expected [B, H, N, D] tensors, got shape %s" % (tuple(t0.shape),))
    for t in ts:
        if t.shape != t0.shape or t.dtype != t0.dtype or t.device != t0.device:
            raise ValueError("q, k, v (and dO) must share shape, dtype and device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [B, H, N, D]")
    return tuple(t0.shape), _dtype_code(t0)


def _on_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("linear attention runs on the GPU only; got a %s tensor"
                             % t.device)


def _check_like(t, like, what):
    """A caller-supplied output must be exactly like `like`: the library
    writes as many elements of that dtype as `like` holds."""
    if t is None:
        return
    if (not isinstance(t, torch.Tensor) or t.shape != like.shape or t.dtype != like.dtype
            or t.device != like.device or not t.is_contiguous()):
        raise ValueError("%s must be a contiguous %s tensor of shape %s on %s"
                         % (what, like.dtype, tuple(like.shape), like.device))


def _check_bytes(t, nbytes, dev, what, dtype=None):
    """A caller-supplied buffer of at least `nbytes` bytes on `dev`
    (contiguous; of `dtype` when given)."""
    if t is None:
        return
    if (not isinstance(t, torch.Tensor) or t.device != dev or not t.is_contiguous()
            or (dtype is not None and t.dtype != dtype)):
        raise ValueError("%s must be a contiguous %stensor on %s"
                         % (what, "" if dtype is None else "%s " % dtype, dev))
    if t.numel() * t.element_size() < nbytes:
        raise ValueError("%s holds %d bytes; this call needs %d"
                         % (what, t.numel() * t.element_size(), nbytes))


def _nbytes(t):
    return t.numel() * t.element_size()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


class KernelTrace:
    """Caller-owned HIP events that the library records around each of its
    kernel launches in one call (see la_forward_traced in include/la.h)."""

    def __init__(self, device, max_launches: int = 8):
        self.max_launches = max_launches
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(2 * max_launches)]
        stream = torch.cuda.current_stream(device)
        for e in self.events:      # torch creates the HIP event on first record
            e.record(stream)
        self._handles = (ctypes.c_void_p * len(self.events))(
            *[ctypes.c_void_p(e.cuda_event) for e in self.events])
        self._names = (ctypes.c_char_p * max_launches)()
        self._n = ctypes.c_int(0)

    def args(self):
        return (ctypes.cast(self._handles, ctypes.c_void_p), len(self.events),
                ctypes.byref(self._n), self._names)

    def names(self):
        return [self._names[i].decode() for i in range(min(self._n.value, self.max_launches))]

    def times_ms(self):
        """Per-launch durations (call after the stream has been synchronised)."""
        return [self.events[2 * i].elapsed_time(self.events[2 * i + 1])
                for i in range(min(self._n.value, self.max_launches))]


def alloc_workspace(B, H, N, D, causal, device, dtype=torch.float32) -> torch.Tensor:
    """Workspace for calls with storage `dtype` (fp32 covers bf16 as well)."""
    return torch.empty(max(workspace_size(B, H, N, D, causal, dtype), 16), dtype=torch.uint8,
                       device=device)


def forward(q, k, v, causal: bool = False, *, return_den: bool = False,
            save_state: bool = False, out=None, state_out=None, workspace=None,
            trace: KernelTrace = None):
    """O = LA(q, k, v).  Returns (O, den or None, state or None).

    ``state_out`` (a float32 CUDA tensor of state_size() bytes) receives the
    saved state; ``save_state=True`` allocates one."""
    (B, H, N, D), dt = _check(q, k, v)
    lib = load_library()
    c = int(bool(causal))
    dev = q.device
    _check_like(out, q, "out")
    _check_bytes(state_out, state_size(B, H, N, D, causal), dev, "state_out", torch.float32)
    _check_bytes(workspace, 0, dev, "workspace")
    _on_gpu(q, out, state_out, workspace)
    o = torch.empty_like(q) if out is None else out
    den = torch.empty((B, H, N), dtype=torch.float32, device=dev) if return_den else None
    state = state_out
    if state is None and save_state:
        state = torch.empty(max(state_size(B, H, N, D, causal) // 4, 4),
                            dtype=torch.float32, device=dev)
    ws = alloc_workspace(B, H, N, D, causal, dev, q.dtype) if workspace is None else workspace
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, N, D, c, dt, _ptr(den), _ptr(state),
            _ptr(ws), _nbytes(ws), _stream(dev))
    if trace is None:
        rc = lib.la_forward(*args)
    else:
        rc = lib.la_forward_traced(*args, *trace.args())
    if rc != 0:
        raise LAError(rc, "la_forward")
    return o, den, state


SCRATCH_BYTES = 64 << 20   # LA_SCRATCH_BYTES: the static workspace of la_forward_noalloc


def forward_noalloc(q, k, v, causal: bool = False, *, out, den_out=None, state_out=None):
    """la_forward_noalloc: the forward pass on the library's static device
    workspace, for callers that cannot allocate (graph capture, serving
    loops).  Every output is the caller's: ``out`` (like q), and optionally
    ``den_out`` (float32 [B, H, N]) and ``state_out`` (state_size() bytes).
    Returns (out, den_out, state_out)."""
    (B, H, N, D), dt = _check(q, k, v)
    lib = load_library()
    dev = q.device
    if out is None:
        raise ValueError("forward_noalloc writes into the caller's out")
    _check_like(out, q, "out")
    if den_out is not None and (den_out.dtype != torch.float32 or den_out.shape != (B, H, N)
                                or den_out.device != dev or not den_out.is_contiguous()):
        raise ValueError("den_out must be a contiguous float32 [B, H, N] tensor on %s" % dev)
    _check_bytes(state_out, state_size(B, H, N, D, causal), dev, "state_out", torch.float32)
    _on_gpu(q, out, den_out, state_out)
    rc = lib.la_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, N, D,
                                int(bool(causal)), dt, _ptr(den_out), _ptr(state_out),
                                _stream(dev))
    if rc != 0:
        raise LAError(rc, "la_forward_noalloc")
    return out, den_out, state_out


def backward(q, k, v, do, causal: bool = False, *, state=None, outs=None,
             workspace=None, trace: KernelTrace = None):
    """Returns (dQ, dK, dV) for the upstream gradient do."""
    (B, H, N, D), dt = _check(q, k, v, do)
    lib = load_library()
    c = int(bool(causal))
    dev = q.device
    if outs is not None:
        if len(outs) != 3:
            raise ValueError("outs must be (dQ, dK, dV)")
        for t, name in zip(outs, ("dQ", "dK", "dV")):
            if t is None:
                raise ValueError("outs: %s is None" % name)
            _check_like(t, q, name)
    # a saved state must be the one the forward wrote for these sizes and
    # this mask (a causal one holds a record per segment)
    _check_bytes(state, state_size(B, H, N, D, causal), dev, "state", torch.float32)
    _check_bytes(workspace, 0, dev, "workspace")
    _on_gpu(q, state, workspace, *(outs or ()))
    if outs is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    else:
        dq, dk, dv = outs
    ws = alloc_workspace(B, H, N, D, causal, dev, q.dtype) if workspace is None else workspace
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, D,
            c, dt, _ptr(state), _ptr(ws), _nbytes(ws), _stream(dev))
    if trace is None:
        rc = lib.la_backward(*args)
    else:
        rc = lib.la_backward_traced(*args, *trace.args())
    if rc != 0:
        raise LAError(rc, "la_backward")
    return dq, dk, dv


def _check_record(r, B, H, D, dev, what):
    if r is None:
        return
    if (not isinstance(r, torch.Tensor) or r.dtype != torch.float32 or r.device != dev
            or not r.is_contiguous() or r.shape != (B, H, D * D + 2 * D)):
        raise ValueError("%s must be a contiguous float32 [B, H, D*D+2*D] tensor on %s"
                         % (what, dev))


def new_record(B, H, D, device) -> torch.Tensor:
    """An uninitialised record tensor [B, H, D*D + 2*D] (float32)."""
    return torch.empty((B, H, D * D + 2 * D), dtype=torch.float32, device=device)


def forward_segment(q, k, v, causal: bool = False, *, carry_in=None, n_carry: int = 0,
                    carry_out=True, compute_out: bool = True, return_den: bool = False,
                    save_state: bool = False, out=None, state_out=None, workspace=None):
    """Forward pass over one piece of a longer sequence (la_forward_segment).

    carry_in: record [B, H, D*D+2D] of the n_carry tokens outside the piece
    that its rows attend to (None = zero).  carry_out: True allocates the
    outgoing record, a tensor receives it, None/False skips it.
    compute_out=False computes only the records.
    Returns (O or None, den or None, carry_out or None, state or None)."""
    (B, H, N, D), dt = _check(q, k, v)
    lib = load_library()
    dev = q.device
    _check_record(carry_in, B, H, D, dev, "carry_in")
    if carry_out is True:
        carry_out = new_record(B, H, D, dev)
    elif carry_out is False:
        carry_out = None
    _check_record(carry_out, B, H, D, dev, "carry_out")
    _check_like(out, q, "out")
    _check_bytes(state_out, state_size(B, H, N, D, causal), dev, "state_out", torch.float32)
    _check_bytes(workspace, 0, dev, "workspace")
    _on_gpu(q, carry_in, carry_out, out, state_out, workspace)
    o = (torch.empty_like(q) if out is None else out) if compute_out else None
    den = torch.empty((B, H, N), dtype=torch.float32, device=dev) if return_den else None
    state = state_out
    if state is None and save_state:
        state = torch.empty(max(state_size(B, H, N, D, causal) // 4, 4),
                            dtype=torch.float32, device=dev)
    ws = alloc_workspace(B, H, N, D, causal, dev, q.dtype) if workspace is None else workspace
    rc = lib.la_forward_segment(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, N, D,
                                int(bool(causal)), dt, _ptr(carry_in), int(n_carry),
                                _ptr(carry_out), _ptr(den), _ptr(state), _ptr(ws), _nbytes(ws),
                                _stream(dev))
    if rc != 0:
        raise LAError(rc, "la_forward_segment")
    return o, den, carry_out, state


def backward_segment(q, k, v, do, causal: bool = False, *, carry_in=None, n_carry: int = 0,
                     gcarry_in=None, gcarry_out=True, compute_kv: bool = True, state=None,
                     outs=None, workspace=None):
    """Backward pass over one piece (la_backward_segment).

    carry_in / n_carry as given to forward_segment (carry_in is read only when
    state is None); gcarry_in: gradient record of the rows outside the piece
    that attend to its keys (None = zero); gcarry_out as carry_out of
    forward_segment.  compute_kv=False computes only dQ and gcarry_out.
    Returns (dQ, dK or None, dV or None, gcarry_out or None)."""
    (B, H, N, D), dt = _check(q, k, v, do)
    lib = load_library()
    dev = q.device
    _check_record(carry_in, B, H, D, dev, "carry_in")
    _check_record(gcarry_in, B, H, D, dev, "gcarry_in")
    if gcarry_out is True:
        gcarry_out = new_record(B, H, D, dev)
    elif gcarry_out is False:
        gcarry_out = None
    _check_record(gcarry_out, B, H, D, dev, "gcarry_out")
    if outs is not None:
        if len(outs) != 3 or outs[0] is None or (outs[1] is None) != (outs[2] is None):
            raise ValueError("outs must be (dQ, dK, dV), with dK and dV both given or both None")
        for t, name in zip(outs, ("dQ", "dK", "dV")):
            _check_like(t, q, name)
    _check_bytes(state, state_size(B, H, N, D, causal), dev, "state", torch.float32)
    _check_bytes(workspace, 0, dev, "workspace")
    _on_gpu(q, carry_in, gcarry_in, gcarry_out, state, workspace, *(outs or ()))
    if outs is None:
        dq = torch.empty_like(q)
        dk, dv = (torch.empty_like(q), torch.empty_like(q)) if compute_kv else (None, None)
    else:
        dq, dk, dv = outs
    ws = alloc_workspace(B, H, N, D, causal, dev, q.dtype) if workspace is None else workspace
    rc = lib.la_backward_segment(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dq), _ptr(dk),
                                 _ptr(dv), B, H, N, D, int(bool(causal)), dt, _ptr(carry_in),
                                 int(n_carry), _ptr(gcarry_in), _ptr(gcarry_out), _ptr(state),
                                 _ptr(ws), _nbytes(ws), _stream(dev))
    if rc != 0:
        raise LAError(rc, "la_backward_segment")
    return dq, dk, dv, gcarry_out


def decode_step(q, k, v, state_in=None, *, state_out=None, counts=None, n_prev: int = 0,
                out=None, return_den: bool = False):
    """One causal decode step (la_decode_step): q, k, v are [B, H, D] (one
    token per head).  state_in: record [B, H, D*D+2D] of the tokens before
    (None = empty prefix); counts: None or a CUDA int64 [B] tensor of the
    tokens before, per sequence (else n_prev for all).
    Returns (o, den or None, state_out)."""
    if q.dim() != 3:
        raise ValueError("decode_step takes [B, H, D] tokens, got shape %s" % (tuple(q.shape),))
    (B, H, _, D), dt = _check(*(t.unsqueeze(2) for t in (q, k, v)))
    lib = load_library()
    dev = q.device
    _check_record(state_in, B, H, D, dev, "state_in")
    if state_out is None:
        state_out = new_record(B, H, D, dev)
    _check_record(state_out, B, H, D, dev, "state_out")
    if counts is not None and (counts.dtype != torch.int64 or counts.device != dev
                               or counts.shape != (B,) or not counts.is_contiguous()):
        raise ValueError("counts must be a contiguous int64 [B] tensor on %s" % dev)
    _check_like(out, q, "out")
    _on_gpu(q, state_in, state_out, counts, out)
    o = torch.empty_like(q) if out is None else out
    den = torch.empty((B, H), dtype=torch.float32, device=dev) if return_den else None
    rc = lib.la_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, D, dt, _ptr(state_in),
                            _ptr(state_out), _ptr(counts), int(n_prev), _ptr(den), _stream(dev))
    if rc != 0:
        raise LAError(rc, "la_decode_step")
    return o, den, state_out


def _layer_dims(x, wqkv, wo, H):
    for t in (x, wqkv, wo):
        if not t.is_contiguous() or t.dtype != x.dtype or t.device != x.device:
            raise ValueError("layer tensors must be contiguous, on one GPU, of one dtype")
    if x.dim() != 3:
        raise ValueError("x must be [B, N, C]")
    B, N, C = x.shape
    if wqkv.dim() != 2 or wqkv.shape[0] != C or wqkv.shape[1] % (3 * H) != 0:
        raise ValueError("wqkv must be [C, 3*H*D]")
    D = wqkv.shape[1] // (3 * H)
    if tuple(wo.shape) != (H * D, C):
        raise ValueError("wo must be [H*D, C]")
    return B, N, C, D, _dtype_code(x)


def layer_sizes(B, N, C, H, D, causal=False, dtype=torch.float32):
    """(saved bytes, workspace bytes) of the layer calls."""
    lib = load_library()
    dt, c = _dtype_of(dtype), int(bool(causal))
    return (int(lib.la_layer_saved_size(B, N, C, H, D, c, dt)),
            int(lib.la_layer_workspace_size(B, N, C, H, D, c, dt)))


def layer_forward(x, wqkv, wo, H: int, causal: bool = False, *, saved=None, out=None,
                  workspace=None, save: bool = True):
    """Y = one linear-attention layer (la_layer_forward).  Returns (Y, saved)
    with `saved` the buffer the backward needs (None when save=False)."""
    B, N, C, D, dt = _layer_dims(x, wqkv, wo, H)
    lib = load_library()
    sb, wb = layer_sizes(B, N, C, H, D, causal, x.dtype)
    _check_like(out, x, "out")
    _check_bytes(saved, sb, x.device, "saved")
    _check_bytes(workspace, 0, x.device, "workspace")
    _on_gpu(x, out, saved, workspace)
    if saved is None and save:
        saved = torch.empty(max(sb, 16), dtype=torch.uint8, device=x.device)
    ws = torch.empty(max(wb, 16), dtype=torch.uint8, device=x.device) if workspace is None \
        else workspace
    y = torch.empty_like(x) if out is None else out
    rc = lib.la_layer_forward(_ptr(x), _ptr(wqkv), _ptr(wo), _ptr(y), B, N, C, H, D,
                              int(bool(causal)), dt, _ptr(saved), _ptr(ws), _nbytes(ws),
                              _stream(x.device))
    if rc != 0:
        raise LAError(rc, "la_layer_forward")
    return y, saved


def layer_backward(x, wqkv, wo, dy, H: int, causal: bool = False, *, saved, outs=None,
                   workspace=None):
    """(dX, dWqkv, dWo) of L = sum dY . Y (la_layer_backward)."""
    B, N, C, D, dt = _layer_dims(x, wqkv, wo, H)
    if dy.shape != x.shape or dy.dtype != x.dtype or not dy.is_contiguous():
        raise ValueError("dy must match x")
    lib = load_library()
    sb, wb = layer_sizes(B, N, C, H, D, causal, x.dtype)
    if saved is None:
        raise ValueError("layer_backward needs the saved buffer of layer_forward")
    _check_bytes(saved, sb, x.device, "saved")
    _check_bytes(workspace, 0, x.device, "workspace")
    if outs is not None:
        if len(outs) != 3:
            raise ValueError("outs must be (dX, dWqkv, dWo)")
        for t, like, name in zip(outs, (x, wqkv, wo), ("dX", "dWqkv", "dWo")):
            if t is None:
                raise ValueError("outs: %s is None" % name)
            _check_like(t, like, name)
    _on_gpu(x, dy, saved, workspace, *(outs or ()))
    ws = torch.empty(max(wb, 16), dtype=torch.uint8, device=x.device) if workspace is None \
        else workspace
    dx, dwqkv, dwo = (torch.empty_like(x), torch.empty_like(wqkv), torch.empty_like(wo)) \
        if outs is None else outs
    rc = lib.la_layer_backward(_ptr(x), _ptr(wqkv), _ptr(wo), _ptr(dy), _ptr(dx), _ptr(dwqkv),
                               _ptr(dwo), B, N, C, H, D, int(bool(causal)), dt, _ptr(saved),
                               _ptr(ws), _nbytes(ws), _stream(x.device))
    if rc != 0:
        raise LAError(rc, "la_layer_backward")
    return dx, dwqkv, dwo


class LinearAttention(torch.autograd.Function):
    """Autograd wrapper: saves q, k, v and the forward's key-value state
    (O(D^2) per head, plus one per segment when causal)."""

    @staticmethod
    def forward(ctx, q, k, v, causal=False):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        o, _, state = forward(q, k, v, causal, save_state=True)
        ctx.save_for_backward(q, k, v, state)
        ctx.causal = causal
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, state = ctx.saved_tensors
        dq, dk, dv = backward(q, k, v, do.contiguous(), ctx.causal, state=state)
        return dq, dk, dv, None


def linear_attention(q, k, v, causal: bool = False):
    return LinearAttention.apply(q, k, v, causal)
