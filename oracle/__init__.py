"""fp64 CPU oracle for Transformer-based linear attention (test infrastructure).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path (the HIP library
and its Python binding) never does.  It shares no code with the HIP path.

The attention arithmetic lives in ``la_oracle.c`` (plain C, fp64).  This
module builds it with gcc, loads it with ctypes and marshals numpy arrays; the
only arithmetic here is the layer around the attention (``layer_forward`` /
``layer_backward``), whose projections are fp64 numpy matrix products.  See the
header of ``la_oracle.c`` for what is computed and which passage of the pages
each step follows ("Transformer Based Linear Attention with Optimized GPU
Kernel Implementation": TL;DR and Figure 1 caption on the sciencestack.ai page;
the reordering and state-update pseudocode in section 2 of the cloud.baidu.com
article).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "la_oracle.c")
_LIB = os.path.join(_HERE, "liblaoracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile la_oracle.c with gcc (no fast-math, OpenMP over heads)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
               "-o", tmp, _SRC]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _bind(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    for name in ("la_oracle_forward_direct", "la_oracle_forward_state"):
        f = getattr(lib, name)
        f.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64, i64, ctypes.c_int]
        f.restype = None
    for name in ("la_oracle_backward_direct", "la_oracle_backward_state"):
        f = getattr(lib, name)
        f.argtypes = [dp, dp, dp, dp, dp, dp, dp, i64, i64, i64, i64,
                      ctypes.c_int]
        f.restype = None
    lib.la_oracle_forward_carry.argtypes = [dp, dp, dp, dp, dp, dp, ctypes.c_double,
                                            dp, i64, i64, i64, i64, ctypes.c_int]
    lib.la_oracle_forward_carry.restype = None
    lib.la_oracle_backward_carry.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp,
                                             ctypes.c_double, dp, dp, i64, i64,
                                             i64, i64, ctypes.c_int]
    lib.la_oracle_backward_carry.restype = None
    lib.la_oracle_max_threads.argtypes = []
    lib.la_oracle_max_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _c64(x) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    if a.ndim != 4:
        raise ValueError("expected a [B,H,N,D] array, got shape %r" % (a.shape,))
    return a


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _check(*arrs):
    shape = arrs[0].shape
    for a in arrs[1:]:
        if a.shape != shape:
            raise ValueError("shape mismatch %r vs %r" % (a.shape, shape))
    return shape


def _forward(name, q, k, v, causal, lib=None):
    q, k, v = _c64(q), _c64(k), _c64(v)
    B, H, N, D = _check(q, k, v)
    o = np.empty_like(q)
    den = np.empty((B, H, N), dtype=np.float64)
    getattr(lib or _load(), name)(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(den),
                           B, H, N, D, int(bool(causal)))
    return o, den


def _backward(name, q, k, v, g, causal, lib=None):
    q, k, v, g = _c64(q), _c64(k), _c64(v), _c64(g)
    B, H, N, D = _check(q, k, v, g)
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    getattr(lib or _load(), name)(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(dq),
                           _ptr(dk), _ptr(dv), B, H, N, D, int(bool(causal)))
    return dq, dk, dv


def _record(rec, B, H, D):
    """A [B,H,D*D+2D] fp64 record, or None."""
    if rec is None:
        return None
    a = np.ascontiguousarray(np.asarray(rec, dtype=np.float64))
    if a.shape != (B, H, D * D + 2 * D):
        raise ValueError("expected a record of shape %r, got %r"
                         % ((B, H, D * D + 2 * D), a.shape))
    return a


def _optr(a):
    return None if a is None else _ptr(a)


def _forward_carry(q, k, v, causal, rec_in, n0, lib=None):
    q, k, v = _c64(q), _c64(k), _c64(v)
    B, H, N, D = _check(q, k, v)
    rec_in = _record(rec_in, B, H, D)
    o = np.empty_like(q)
    den = np.empty((B, H, N), dtype=np.float64)
    rec_out = np.empty((B, H, D * D + 2 * D), dtype=np.float64)
    (lib or _load()).la_oracle_forward_carry(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(den), _optr(rec_in), float(n0),
        _ptr(rec_out), B, H, N, D, int(bool(causal)))
    return o, den, rec_out


def _backward_carry(q, k, v, g, causal, rec_in, n0, grec_in, lib=None):
    q, k, v, g = _c64(q), _c64(k), _c64(v), _c64(g)
    B, H, N, D = _check(q, k, v, g)
    rec_in, grec_in = _record(rec_in, B, H, D), _record(grec_in, B, H, D)
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    grec_out = np.empty((B, H, D * D + 2 * D), dtype=np.float64)
    (lib or _load()).la_oracle_backward_carry(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(dq), _ptr(dk), _ptr(dv),
        _optr(rec_in), float(n0), _optr(grec_in), _ptr(grec_out), B, H, N, D,
        int(bool(causal)))
    return dq, dk, dv, grec_out


def forward_direct(q, k, v, causal=False):
    """O(N^2 D) definition: returns (O, den) as fp64 arrays."""
    return _forward("la_oracle_forward_direct", q, k, v, causal)


def forward_state(q, k, v, causal=False):
    """O(N D^2) state form (reordered products / token recurrence)."""
    return _forward("la_oracle_forward_state", q, k, v, causal)


def backward_direct(q, k, v, g, causal=False):
    """O(N^2 D) analytical gradients: returns (dQ, dK, dV)."""
    return _backward("la_oracle_backward_direct", q, k, v, g, causal)


def backward_state(q, k, v, g, causal=False):
    """O(N D^2) gradients through the forward and gradient states."""
    return _backward("la_oracle_backward_state", q, k, v, g, causal)


def forward_carry(q, k, v, causal=False, rec_in=None, n0=0):
    """State form over one piece of a longer sequence.  rec_in is the record
    [S | z | u] ([B,H,D*D+2D]) of n0 tokens outside the piece whose keys every
    row of the piece sees (causal: the tokens before it; non-causal: the rest
    of the sequence), or None.  Returns (O, den, rec_out) with rec_out the
    record of those tokens plus the piece's own."""
    return _forward_carry(q, k, v, causal, rec_in, n0)


def backward_carry(q, k, v, g, causal=False, rec_in=None, n0=0, grec_in=None):
    """Gradients of one piece.  rec_in, n0 as for forward_carry; grec_in is
    the gradient record [R | r | t] of the rows outside the piece that see
    its keys (causal: the rows after it; non-causal: the other rows), or
    None.  Returns (dQ, dK, dV, grec_out) with grec_out = grec_in plus the
    piece's own rows' record."""
    return _backward_carry(q, k, v, g, causal, rec_in, n0, grec_in)


def _split_heads(t, H, D):
    B, N, _ = t.shape
    return np.ascontiguousarray(t.reshape(B, N, H, D).transpose(0, 2, 1, 3))


def _merge_heads(t):
    B, H, N, D = t.shape
    return np.ascontiguousarray(t.transpose(0, 2, 1, 3).reshape(B, N, H * D))


def layer_forward(x, wqkv, wo, H, D, causal=False):
    """One linear-attention layer (shd-paper.top digest, technical-framework
    paragraph 技术框架:
    the input rows pass through a linear map, linear attention forms the
    context rows, a further map follows; the plainest reading is a query /
    key / value projection and an output projection without biases):
    [Q | K | V] = X Wqkv, O_h = LA(Q_h, K_h, V_h), Y = [O_1 .. O_H] Wo.
    x [B, N, C], wqkv [C, 3HD], wo [HD, C]; returns Y [B, N, C] in fp64."""
    x, wqkv, wo = (np.asarray(a, dtype=np.float64) for a in (x, wqkv, wo))
    HD = H * D
    qkv = np.matmul(x, wqkv)
    q, k, v = (_split_heads(qkv[..., j * HD:(j + 1) * HD], H, D) for j in range(3))
    o, _ = forward_state(q, k, v, causal)
    return np.matmul(_merge_heads(o), wo)


def layer_backward(x, wqkv, wo, dy, H, D, causal=False):
    """Gradients of L = sum dY . Y for layer_forward, by the chain rule
    through the two products and the attention's own backward:
    dWo = O^T dY, dO = dY Wo^T, (dQ, dK, dV) = LA backward, dWqkv = X^T dQKV,
    dX = dQKV Wqkv^T (sums over the batch).  Returns (dX, dWqkv, dWo)."""
    x, wqkv, wo, dy = (np.asarray(a, dtype=np.float64) for a in (x, wqkv, wo, dy))
    HD = H * D
    qkv = np.matmul(x, wqkv)
    q, k, v = (_split_heads(qkv[..., j * HD:(j + 1) * HD], H, D) for j in range(3))
    o, _ = forward_state(q, k, v, causal)
    orows = _merge_heads(o)
    dwo = np.einsum("bni,bnc->ic", orows, dy)
    do = _split_heads(np.matmul(dy, wo.T), H, D)
    dq, dk, dv = backward_state(q, k, v, do, causal)
    dqkv = np.concatenate([_merge_heads(t) for t in (dq, dk, dv)], axis=-1)
    dwqkv = np.einsum("bnc,bnj->cj", x, dqkv)
    dx = np.matmul(dqkv, wqkv.T)
    return dx, dwqkv, dwo


def max_threads() -> int:
    return int(_load().la_oracle_max_threads())


class Variant:
    """The same API bound to another build of la_oracle.c (used by the test
    that plants mistakes in a copy of the oracle source to show that the pins
    catch them)."""

    def __init__(self, so_path):
        self._lib = _bind(ctypes.CDLL(so_path))

    def forward_direct(self, q, k, v, causal=False):
        return _forward("la_oracle_forward_direct", q, k, v, causal, self._lib)

    def forward_state(self, q, k, v, causal=False):
        return _forward("la_oracle_forward_state", q, k, v, causal, self._lib)

    def backward_direct(self, q, k, v, g, causal=False):
        return _backward("la_oracle_backward_direct", q, k, v, g, causal, self._lib)

    def backward_state(self, q, k, v, g, causal=False):
        return _backward("la_oracle_backward_state", q, k, v, g, causal, self._lib)

    def forward_carry(self, q, k, v, causal=False, rec_in=None, n0=0):
        return _forward_carry(q, k, v, causal, rec_in, n0, self._lib)

    def backward_carry(self, q, k, v, g, causal=False, rec_in=None, n0=0, grec_in=None):
        return _backward_carry(q, k, v, g, causal, rec_in, n0, grec_in, self._lib)


def build_variant(src_text: str, out_dir: str) -> "Variant":
    """Compile C source text (a modified copy of la_oracle.c) and bind it."""
    src = os.path.join(out_dir, "variant.c")
    so = os.path.join(out_dir, "libvariant.so")
    with open(src, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                    "-ffp-contract=off", "-w", "-o", so, src], check=True)
    return Variant(so)


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()
