"""C-ABI checks that need no GPU: the library loads, exports every function
that include/la.h declares, and rejects bad arguments on the host before any
launch.  The argument-validation cases pass host addresses as stand-ins for
device pointers, so they only run where no GPU is visible (a validation bug
there could otherwise launch a kernel on them)."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

import linear_attention_transformer_amd as la

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "la.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(la_[a-z_]+)\s*\(", text)))


def test_library_built_and_loads():
    assert os.path.exists(la.LIB_PATH)
    la.load_library()


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert {"la_forward", "la_backward", "la_workspace_size", "la_state_size",
            "la_status_string", "la_num_segments"} <= set(names)
    lib = ctypes.CDLL(la.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", la.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (la_\w+)", out))
    assert set(names) <= exported


def test_status_strings():
    for code, name in la.STATUS.items():
        assert la.status_string(code).startswith(name)
    assert la.status_string(99) == "unknown la_status"


def test_sizes():
    B, H, N, D = 4, 16, 4096, 128
    ns = la.num_segments(B, H, N, D)
    assert ns == 8
    ps = D * D + 2 * D
    assert la.state_size(B, H, N, D, False) == B * H * ps * 4
    assert la.state_size(B, H, N, D, True) == B * H * ns * ps * 4
    ws = la.workspace_size(B, H, N, D, True)
    # workspace is O(B H (segments D^2 + N)): far below one [B,H,N,D] tensor
    # once N >> D; here it must stay below the four fp32 inputs
    assert 0 < ws < 4 * B * H * N * D * 4
    assert la.workspace_size(0, 16, 4096, 128) == 0
    assert la.workspace_size(4, 16, 4096, 300) == 0      # unsupported D
    assert la.workspace_size(4, 16, 4096, 0) == 0
    # padded head sizes (between the native 32, 64, 128, 256) need room for
    # seven padded tensors on top of the native workspace
    nat = la.workspace_size(B, H, N, 64)
    pad = B * H * N * 64
    assert la.workspace_size(B, H, N, 48) >= nat + 7 * pad * 4
    for dt in (torch.bfloat16, torch.float16):
        assert la.workspace_size(B, H, N, 64, dtype=dt) == nat
        assert nat + 7 * pad * 2 <= la.workspace_size(B, H, N, 48, dtype=dt) < \
            la.workspace_size(B, H, N, 48)
    # heads of D <= 16 run at width 16 on the caller's rows: records of width
    # 16, and a workspace without padded tensors (below one [B,H,N,16] fp32)
    ns16 = la.num_segments(B, H, N, 6)
    for d in (1, 6, 16):
        assert la.num_segments(B, H, N, d) == ns16
        assert la.state_size(B, H, N, d, False) == B * H * (16 * 16 + 2 * 16) * 4
        assert la.state_size(B, H, N, d, True) == B * H * ns16 * (16 * 16 + 2 * 16) * 4
    for d in (1, 6, 16):
        assert 0 < la.workspace_size(B, H, N, d) < B * H * N * 16 * 4
    assert la.workspace_size(4, 16, -1, 128) == 0
    # short sequences: segments of at least 256 rows where that still leaves
    # one workgroup per CU (64 heads), else the plan's shorter segments
    assert la.num_segments(4, 16, 1024, 128) == 4
    assert la.num_segments(4, 16, 640, 128) == 5
    assert la.num_segments(1, 4, 1024, 128) == 16
    # segments grow with N, never exceed the 64-row chunks
    for n in (1, 63, 64, 65, 1000, 131072):
        s = la.num_segments(1, 1, n, 64)
        assert 1 <= s <= max(1, (n + 63) // 64)


needs_no_gpu = pytest.mark.skipif(torch.cuda.is_available(),
                                  reason="host-only validation with stand-in pointers")


@needs_no_gpu
def test_host_validation_rejects_before_launch():
    lib = la.load_library()
    buf = (ctypes.c_char * (1 << 20))()
    base = ctypes.addressof(buf)
    a16 = (base + 15) & ~15
    P = lambda off=0: ctypes.c_void_p(a16 + off)
    B, H, N, D = 1, 2, 8, 16
    ws = la.workspace_size(B, H, N, D, False)
    tb = B * H * N * D * 4
    f = lib.la_forward
    # dtype, causal, sizes, D
    assert f(P(), P(tb), P(2 * tb), P(3 * tb), B, H, N, D, 0, 7, None, None, P(4 * tb), ws, None) == 3
    assert f(P(), P(tb), P(2 * tb), P(3 * tb), B, H, N, D, 2, 0, None, None, P(4 * tb), ws, None) == 4
    assert f(P(), P(tb), P(2 * tb), P(3 * tb), B, H, -1, D, 0, 0, None, None, P(4 * tb), ws, None) == 2
    assert f(P(), P(tb), P(2 * tb), P(3 * tb), B, H, N, 300, 0, 0, None, None, P(4 * tb), ws, None) == 4
    assert f(P(), P(tb), P(2 * tb), P(3 * tb), B, H, N, 0, 0, 0, None, None, P(4 * tb), ws, None) == 4
    # a padded head size (D = 6) with too small a workspace, in fp32 and fp16
    assert f(P(), P(tb), P(2 * tb), P(3 * tb), B, H, N, 6, 0, 0, None, None, P(4 * tb), 4096,
             None) == 5
    assert f(P(), P(tb), P(2 * tb), P(3 * tb), B, H, N, 6, 0, 2, None, None, P(4 * tb), 4096,
             None) == 5
    assert f(P(), P(tb), P(2 * tb), P(3 * tb), 1 << 40, 1 << 40, N, D, 0, 0, None, None,
             P(4 * tb), ws, None) == 2
    # empty problem is a no-op even with NULL pointers
    assert f(None, None, None, None, B, H, 0, D, 0, 0, None, None, None, 0, None) == 0
    # NULL, workspace, alignment, aliasing
    assert f(None, P(tb), P(2 * tb), P(3 * tb), B, H, N, D, 0, 0, None, None, P(4 * tb), ws, None) == 1
    assert f(P(), P(tb), P(2 * tb), P(3 * tb), B, H, N, D, 0, 0, None, None, P(4 * tb), ws - 4, None) == 5
    assert f(P(4), P(tb), P(2 * tb), P(3 * tb), B, H, N, D, 0, 0, None, None, P(4 * tb), ws, None) == 7
    assert f(P(), P(tb), P(2 * tb), P(0), B, H, N, D, 0, 0, None, None, P(4 * tb), ws, None) == 6
    assert f(P(), P(tb), P(2 * tb), P(3 * tb), B, H, N, D, 0, 0, None, None, P(3 * tb), ws, None) == 6
    assert f(P(), P(tb), P(2 * tb), P(3 * tb), B, H, N, D, 0, 0, ctypes.c_void_p(a16 + 3 * tb + 16),
             None, P(4 * tb), ws, None) == 6
    g = lib.la_backward
    args = lambda q, gw: (P(q), P(tb), P(2 * tb), P(3 * tb), P(4 * tb), P(5 * tb), P(6 * tb),
                          B, H, N, D, 0, 0, None, P(7 * tb), gw)
    assert g(*args(0, ws - 16), None) == 5
    assert g(*args(8, ws), None) == 7
    assert g(P(), P(tb), P(2 * tb), P(3 * tb), P(4 * tb), P(4 * tb), P(6 * tb), B, H, N, D, 0, 0,
             None, P(7 * tb), ws, None) == 6
    assert g(P(), P(tb), P(2 * tb), P(3 * tb), P(4 * tb), P(5 * tb), P(6 * tb), B, H, N, D, 0, 0,
             P(4 * tb), P(7 * tb), ws, None) == 6
    assert g(P(), P(tb), P(2 * tb), None, P(4 * tb), P(5 * tb), P(6 * tb), B, H, N, D, 0, 0,
             None, P(7 * tb), ws, None) == 1
    # la_backward needs dK and dV
    assert g(P(), P(tb), P(2 * tb), P(3 * tb), P(4 * tb), None, None, B, H, N, D, 0, 0,
             None, P(7 * tb), ws, None) == 1


@needs_no_gpu
def test_host_validation_segment_calls():
    """The carried-state calls reject bad records and counts before launch."""
    lib = la.load_library()
    buf = (ctypes.c_char * (1 << 21))()
    a16 = (ctypes.addressof(buf) + 15) & ~15
    P = lambda off=0: ctypes.c_void_p(a16 + off)
    B, H, N, D = 1, 2, 8, 16
    ws = la.workspace_size(B, H, N, D, True)
    tb = B * H * N * D * 4
    rb = la.record_size(B, H, D)
    assert rb == B * H * (D * D + 2 * D) * 4
    assert la.record_size(1, 1, 300) == 0 and la.record_size(-1, 1, 16) == 0
    assert la.record_size(1, 1, 6) == 48 * 4
    W, CI, CO = 4 * tb, 4 * tb + ws + 256, 4 * tb + ws + 256 + rb + 256
    f = lib.la_forward_segment

    def fa(o=P(3 * tb), cin=P(CI), n=5, cout=P(CO), den=None, st=None, N_=N):
        return f(P(), P(tb), P(2 * tb), o, B, H, N_, D, 1, 0, cin, n, cout, den, st, P(W), ws,
                 None)

    assert fa(n=-1) == 2
    assert fa(n=(1 << 40) + 1) == 2
    assert fa(cout=P(CI + 16)) == 6              # carry_out overlaps carry_in
    assert fa(cout=P(0)) == 6                    # carry_out overlaps Q
    assert fa(cin=P(3 * tb)) == 6                # O overlaps carry_in
    assert fa(cout=P(CO + 4)) == 7
    assert fa(cin=P(CI + 8)) == 7
    assert fa(o=None, cout=None) == 1            # nothing would receive a result
    assert fa(o=None, den=P(CO + rb + 256)) == 1  # den needs O
    assert fa(N_=0, cout=P(CI + 16)) == 6        # zero tokens: pass-through checks still apply
    assert fa(N_=0, cout=P(CO + 4)) == 7
    g = lib.la_backward_segment

    def ga(dk=P(5 * tb), dv=P(6 * tb), gin=P(CI), gout=P(CO), n=5):
        return g(P(), P(tb), P(2 * tb), P(3 * tb), P(4 * tb), dk, dv, B, H, N, D, 1, 0, None, n,
                 gin, gout, None, P(7 * tb), ws, None)

    ws_b = 7 * tb
    CI, CO = ws_b + ws + 256, ws_b + ws + 256 + rb + 256
    assert ga(gin=P(CI), gout=P(CO), n=-3) == 2
    assert ga(dk=None, gin=P(CI), gout=P(CO)) == 1     # dK without dV
    assert ga(dv=None, gin=P(CI), gout=P(CO)) == 1
    assert ga(gin=P(CI), gout=P(CI + 32)) == 6         # gcarry_out overlaps gcarry_in
    assert ga(gin=P(CI), gout=P(4 * tb)) == 6          # gcarry_out overlaps dQ
    assert ga(gin=P(CI + 4), gout=P(CO)) == 7


@needs_no_gpu
def test_host_validation_decode_step():
    lib = la.load_library()
    buf = (ctypes.c_char * (1 << 20))()
    a16 = (ctypes.addressof(buf) + 15) & ~15
    P = lambda off=0: ctypes.c_void_p(a16 + off)
    B, H, D = 2, 2, 16
    tb = B * H * D * 4
    rb = la.record_size(B, H, D)
    SI, SO = 4 * tb, 4 * tb + rb + 256
    d = lib.la_decode_step

    def da(q=P(0), o=P(3 * tb), si=P(SI), so=P(SO), counts=None, n=3, dt=0, D_=D):
        return d(q, P(tb), P(2 * tb), o, B, H, D_, dt, si, so, counts, n, None, None)

    assert da(dt=5) == 3
    assert da(D_=300) == 4
    assert da(D_=0) == 4
    assert da(n=-1) == 2
    assert da(q=None) == 1
    assert da(so=None) == 1
    assert da(so=P(SI + 64)) == 6          # state_out overlaps state_in
    assert da(o=P(tb)) == 6                # o overlaps k
    assert da(so=P(SO + 8)) == 7
    assert da(counts=P(SO + rb + 260)) == 7


def test_python_side_refuses_cpu_tensors():
    q = torch.zeros(1, 1, 4, 16)
    with pytest.raises(ValueError):
        la.forward(q, q, q)


@needs_no_gpu
def test_host_validation_layer_calls():
    """The layer calls reject bad shapes, pointers and workspaces before
    touching rocBLAS or launching anything."""
    lib = la.load_library()
    B, N, C, H, D = 1, 8, 16, 2, 8
    sb = lib.la_layer_saved_size(B, N, C, H, D, 0, 0)
    wb = lib.la_layer_workspace_size(B, N, C, H, D, 0, 0)
    assert sb > 0 and wb > sb
    assert lib.la_layer_workspace_size(B, N, C, H, 300, 0, 0) == 0
    assert lib.la_layer_saved_size(B, N, C, H, D, 0, 9) == 0
    # bf16 needs half the fp32 tensors (plus the fixed rocBLAS scratch)
    assert lib.la_layer_workspace_size(B, N, C, H, D, 0, 1) < wb
    buf = (ctypes.c_char * (wb + sb + (1 << 20)))()
    a16 = (ctypes.addressof(buf) + 255) & ~255
    P = lambda off=0: ctypes.c_void_p(a16 + off)
    xb, wq, wo = B * N * C * 4, C * 3 * H * D * 4, H * D * C * 4
    X, WQ, WO, Y = 0, 4096, 8192, 12288
    SV, WS = 16384, 16384 + ((sb + 255) // 256) * 256
    f = lib.la_layer_forward

    def fa(x=P(X), y=P(Y), b=B, n=N, c=C, h=H, d=D, causal=0, dt=0, sv=P(SV), ws=P(WS), wsb=wb):
        return f(x, P(WQ), P(WO), y, b, n, c, h, d, causal, dt, sv, ws, wsb, None)

    assert fa(dt=7) == 3
    assert fa(causal=2) == 4 and fa(d=0) == 4 and fa(d=300) == 4
    assert fa(b=-1) == 2
    assert fa(h=0) == 2
    assert fa(x=None) == 1 and fa(ws=None) == 1
    assert fa(wsb=wb - sb - 1) == 5                 # with a saved buffer
    assert fa(x=P(X + 4)) == 7
    assert fa(y=P(X + 16)) == 6                     # Y overlaps X
    assert fa(b=0) == 0 and fa(c=0) == 0            # empty: nothing to do
    g = lib.la_layer_backward

    def ga(dx=P(X + xb + 1024), sv=P(SV), wsb=wb):
        return g(P(X), P(WQ), P(WO), P(Y), dx, P(WS + wb), P(WS + wb + wq + 256), B, N, C, H, D,
                 0, 0, sv, P(WS), wsb, None)

    assert ga(sv=None) == 1
    assert ga(wsb=1024) == 5
    assert ga(dx=P(Y)) == 6                         # dX overlaps dY
    assert xb <= 4096 and wq <= 4096 and wo <= 4096
