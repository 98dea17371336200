"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/sa.h, and host-side validation returns the documented
status codes synchronously (no kernel is launched on any error path)."""

import ctypes
import os
import re

import numpy as np
import pytest

from recommender_ultra_long_amd import sa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "sa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sa_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = sa.load()
    names = _declared_functions()
    assert set(names) == set(sa.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_version_and_status_strings():
    assert sa.version() == 10000
    for code in range(10):
        s = sa.status_string(code)
        assert s.startswith("SA_")
    assert sa.status_string(123) == "SA_ERR_UNKNOWN"


def _p(**kw):
    base = dict(batch=2, k=64, d=32, total_tokens=100, dtype=sa.SA_F32, mass_norm=False)
    base.update(kw)
    return sa.make_problem(base["batch"], base["k"], base["d"], base["total_tokens"], base["dtype"],
                           base["mass_norm"])


def test_validate_shapes_and_dtypes():
    assert sa.validate(_p()) == sa.SA_OK
    assert sa.validate(_p(dtype=sa.SA_BF16, d=128, k=1024)) == sa.SA_OK
    assert sa.validate(_p(k=2048)) == sa.SA_OK
    assert sa.validate(_p(k=0)) == sa.SA_ERR_BAD_SHAPE
    assert sa.validate(_p(k=2049)) == sa.SA_ERR_BAD_SHAPE
    assert sa.validate(_p(d=48)) == sa.SA_ERR_BAD_SHAPE
    assert sa.validate(_p(d=256)) == sa.SA_ERR_BAD_SHAPE
    assert sa.validate(_p(batch=0)) == sa.SA_ERR_BAD_SHAPE
    assert sa.validate(_p(total_tokens=-1)) == sa.SA_ERR_BAD_SHAPE
    assert sa.validate(_p(total_tokens=1 << 36)) == sa.SA_ERR_BAD_SHAPE
    assert sa.validate(_p(dtype=7)) == sa.SA_ERR_BAD_DTYPE
    pr = _p()
    pr.flags = sa.SA_FLAG_MASS_NORM | sa.SA_FLAG_PER_USER_PROTOTYPES
    assert sa.validate(pr) == sa.SA_OK
    pr.flags = sa.SA_FLAG_TOKEN_WISE
    assert sa.validate(pr) == sa.SA_OK
    # token-wise weights already sum to one; that variant takes a shared table
    pr.flags = sa.SA_FLAG_TOKEN_WISE | sa.SA_FLAG_MASS_NORM
    assert sa.validate(pr) == sa.SA_ERR_UNSUPPORTED
    pr.flags = sa.SA_FLAG_TOKEN_WISE | sa.SA_FLAG_PER_USER_PROTOTYPES
    assert sa.validate(pr) == sa.SA_ERR_UNSUPPORTED
    pr.flags = 8
    assert sa.validate(pr) == sa.SA_ERR_UNSUPPORTED


def test_validate_host_offsets():
    assert sa.validate(_p(), np.array([0, 40, 100])) == sa.SA_OK
    assert sa.validate(_p(), np.array([0, 0, 100])) == sa.SA_OK
    assert sa.validate(_p(), np.array([1, 40, 100])) == sa.SA_ERR_BAD_OFFSETS
    assert sa.validate(_p(), np.array([0, 40, 99])) == sa.SA_ERR_BAD_OFFSETS
    assert sa.validate(_p(), np.array([0, 60, 40])) == sa.SA_ERR_BAD_OFFSETS


def test_workspace_size():
    f = sa.workspace_size(_p(), sa.SA_OP_FORWARD)
    b = sa.workspace_size(_p(), sa.SA_OP_BACKWARD)
    assert f > 0 and b > 0 and f % 256 == 0 and b % 256 == 0
    # per-user tables: the forward needs nothing more; the backward holds a
    # padded copy of every user's table and a dP partial per piece
    pu = _p()
    pu.flags = sa.SA_FLAG_PER_USER_PROTOTYPES
    assert sa.workspace_size(pu, sa.SA_OP_FORWARD) == f
    assert sa.workspace_size(pu, sa.SA_OP_BACKWARD) > b
    assert sa.workspace_size(_p(k=0), sa.SA_OP_FORWARD) == 0
    assert sa.workspace_size(_p(), 5) == 0
    # grows with the token count (the per-token lse and backward buffers)
    assert sa.workspace_size(_p(total_tokens=10000), 0) > f
    assert sa.workspace_size(_p(total_tokens=10000), 1) > b


def _call_forward(pr, off=1, X=1, P=1, S=1, lse=0, mass=0, ws=1, ws_bytes=1 << 30):
    # Fake but 256-aligned addresses: every call below must fail validation
    # before any pointer is dereferenced or any kernel enqueued.
    lib = sa.load()
    a = lambda v: ctypes.c_void_p(v * 4096) if v else None
    return lib.sa_forward(ctypes.byref(pr), a(off), a(X), a(P), a(S), a(lse), a(mass), a(ws),
                          ctypes.c_size_t(ws_bytes), None)


def _call_backward(pr, off=1, X=1, P=1, dS=1, lse=0, S=0, mass=0, dX=1, dP=1, ws=1,
                   ws_bytes=1 << 30):
    lib = sa.load()
    a = lambda v: ctypes.c_void_p(v * 4096) if v else None
    return lib.sa_backward(ctypes.byref(pr), a(off), a(X), a(P), a(dS), a(lse), a(S), a(mass),
                           a(dX), a(dP), a(ws), ctypes.c_size_t(ws_bytes), None)


def test_forward_argument_errors_are_synchronous():
    pr = _p()
    assert _call_forward(pr, off=0) == sa.SA_ERR_NULL_ARG
    assert _call_forward(pr, X=0) == sa.SA_ERR_NULL_ARG
    assert _call_forward(pr, P=0) == sa.SA_ERR_NULL_ARG
    assert _call_forward(pr, S=0) == sa.SA_ERR_NULL_ARG
    assert _call_forward(pr, ws=0) == sa.SA_ERR_NULL_ARG
    assert _call_forward(pr, ws_bytes=16) == sa.SA_ERR_WORKSPACE_TOO_SMALL
    assert _call_forward(_p(k=0)) == sa.SA_ERR_BAD_SHAPE
    assert _call_forward(_p(dtype=5)) == sa.SA_ERR_BAD_DTYPE
    lib = sa.load()
    mis = lib.sa_forward(ctypes.byref(pr), ctypes.c_void_p(4096), ctypes.c_void_p(4096 + 8),
                         ctypes.c_void_p(8192), ctypes.c_void_p(12288), None, None,
                         ctypes.c_void_p(16384), ctypes.c_size_t(1 << 30), None)
    assert mis == sa.SA_ERR_MISALIGNED
    mis = lib.sa_forward(ctypes.byref(pr), ctypes.c_void_p(4096 + 4), ctypes.c_void_p(8192),
                         ctypes.c_void_p(8192), ctypes.c_void_p(12288), None, None,
                         ctypes.c_void_p(16384), ctypes.c_size_t(1 << 30), None)
    assert mis == sa.SA_ERR_MISALIGNED


def test_backward_argument_errors_are_synchronous():
    pr = _p()
    assert _call_backward(pr, dS=0) == sa.SA_ERR_NULL_ARG
    assert _call_backward(pr, dX=0) == sa.SA_ERR_NULL_ARG
    assert _call_backward(pr, dP=0) == sa.SA_ERR_NULL_ARG
    assert _call_backward(pr, ws_bytes=16) == sa.SA_ERR_WORKSPACE_TOO_SMALL
    prm = _p(mass_norm=True)
    assert _call_backward(prm) == sa.SA_ERR_NULL_ARG            # S and mass required
    assert _call_backward(prm, S=2) == sa.SA_ERR_NULL_ARG
    assert _call_backward(_p(d=40)) == sa.SA_ERR_BAD_SHAPE


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(sa, "_lib", None)
    monkeypatch.setattr(sa, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        sa.load()


def test_fold_argument_errors_are_synchronous():
    lib = sa.load()
    buf = ctypes.create_string_buffer(64)   # host memory, 16-byte alignment not required here
    vp = ctypes.c_void_p
    # backward workspace: Q and dQ (k x d) and two d x d partial sums per
    # 128-row slice
    assert lib.sa_fold_workspace_size(1024, 128) == (2 * 1024 * 128 + 2 * 8 * 128 * 128) * 4
    assert lib.sa_fold_workspace_size(129, 32) == (2 * 129 * 32 + 2 * 2 * 32 * 32) * 4
    assert lib.sa_fold_workspace_size(0, 128) == 0
    assert lib.sa_fold_workspace_size(1024, 96) == 0
    # stacked per-user tables: up to 2^24 rows, at most 256 slices
    assert lib.sa_fold_workspace_size(4096, 64) == (2 * 4096 * 64 + 2 * 32 * 64 * 64) * 4
    assert lib.sa_fold_workspace_size(256 * 1024, 128) == (2 * 262144 * 128 + 2 * 256 * 128 * 128) * 4
    assert lib.sa_fold_workspace_size(40000, 128) == (2 * 40000 * 128 + 2 * 157 * 128 * 128) * 4
    assert lib.sa_fold_workspace_size((1 << 24) + 1, 32) == 0
    nul = vp(None)
    # shape and dtype errors come first, with null pointers (no HIP call)
    assert lib.sa_fold_prototypes(0, 128, sa.SA_BF16, nul, nul, nul, nul, nul) == sa.SA_ERR_BAD_SHAPE
    assert lib.sa_fold_prototypes(64, 48, sa.SA_BF16, nul, nul, nul, nul, nul) == sa.SA_ERR_BAD_SHAPE
    assert lib.sa_fold_prototypes(64, 64, 7, nul, nul, nul, nul, nul) == sa.SA_ERR_BAD_DTYPE
    assert lib.sa_fold_prototypes(64, 64, sa.SA_F32, nul, nul, nul, nul, nul) == sa.SA_ERR_NULL_ARG
    assert lib.sa_fold_prototypes_backward(64, 64, sa.SA_F32, nul, nul, nul, nul, nul, nul, nul, nul, 0,
                                           nul) == sa.SA_ERR_NULL_ARG
    # misaligned pointer
    odd = vp(ctypes.addressof(buf) | 1)
    assert lib.sa_fold_prototypes(64, 64, sa.SA_F32, odd, odd, odd, odd, nul) == sa.SA_ERR_MISALIGNED
    assert lib.sa_fold_prototypes_backward(64, 64, sa.SA_F32, odd, odd, odd, odd, odd, odd, odd, odd,
                                           1 << 20, nul) == sa.SA_ERR_MISALIGNED
    # workspace too small (aligned host addresses; the size check precedes any launch)
    al = vp((ctypes.addressof(buf) + 15) & ~15)
    assert lib.sa_fold_prototypes_backward(64, 64, sa.SA_F32, al, al, al, al, al, al, al, al, 16,
                                           nul) == sa.SA_ERR_WORKSPACE_TOO_SMALL


def test_stca_argument_errors_are_synchronous():
    # Reordered single-query STCA (Eq. 24): shape, pointer, alignment and
    # workspace checks all return before any HIP call, so they run on the CPU.
    lib = sa.load()
    a256 = lambda v: (v + 255) // 256 * 256
    D, h, R = 1024, 16, 40
    want = (a256(R * D * 4) + a256(R * h * D * 4) + a256(R * h * D * 2) + a256(R * h * D * 4)
            + a256(R * h * 4))
    assert lib.sa_stca_workspace_size(D, h, R) == want
    assert lib.sa_stca_workspace_size(128, 4, R) == 0          # D not in {256, 512, 1024}
    assert lib.sa_stca_workspace_size(256, 3, R) == 0          # heads must divide D
    assert lib.sa_stca_workspace_size(256, 0, R) == 0
    assert lib.sa_stca_workspace_size(256, 4, -1) == 0
    buf = ctypes.create_string_buffer(256)
    al = (ctypes.addressof(buf) + 15) & ~15
    vp = ctypes.c_void_p
    ok = vp(al)
    nul = vp(None)

    def call(B=2, D=256, h=4, L=10, R=3, x_off=ok, t_off=ok, X=ok, Q=ok, Wq=ok, Wk=ok, Wv=ok,
             o=ok, lse=nul, ws=ok, ws_bytes=1 << 40):
        return lib.sa_stca_attention(B, D, h, L, R, x_off, t_off, X, Q, Wq, Wk, Wv, o, lse, ws,
                                     ctypes.c_size_t(ws_bytes), nul)

    assert call(D=128) == sa.SA_ERR_BAD_SHAPE
    assert call(h=5) == sa.SA_ERR_BAD_SHAPE
    assert call(B=0) == sa.SA_ERR_BAD_SHAPE
    assert call(L=-1) == sa.SA_ERR_BAD_SHAPE
    assert call(x_off=nul) == sa.SA_ERR_NULL_ARG
    assert call(Wk=nul) == sa.SA_ERR_NULL_ARG
    assert call(ws=nul) == sa.SA_ERR_NULL_ARG
    assert call(X=nul) == sa.SA_ERR_NULL_ARG                 # rows present, no X
    assert call(Q=nul) == sa.SA_ERR_NULL_ARG                 # targets present, no queries
    assert call(o=nul) == sa.SA_ERR_NULL_ARG
    odd = vp(al + 4)
    assert call(Wq=odd) == sa.SA_ERR_MISALIGNED
    assert call(t_off=vp(al + 4)) == sa.SA_ERR_MISALIGNED    # int64 offsets: 8-byte alignment
    assert call(ws_bytes=16) == sa.SA_ERR_WORKSPACE_TOO_SMALL
    # no targets: nothing to compute, nothing enqueued
    assert call(R=0, Q=nul, o=nul) == sa.SA_OK


def test_loaded_library_is_the_selected_build():
    # SA_LIBRARY_PATH selects the host-side AddressSanitizer build in
    # test_abi_asan.py; otherwise the in-tree library is loaded.
    want = os.environ.get("SA_LIBRARY_PATH") or os.path.join(ROOT, "recommender_ultra_long_amd",
                                                              "libsa.so")
    assert os.path.samefile(sa.lib_path(), want)


def test_block_argument_errors_are_synchronous():
    lib = sa.load()
    buf = ctypes.create_string_buffer(1024)
    al = (ctypes.addressof(buf) + 255) & ~255
    vp = ctypes.c_void_p
    ok, nul = vp(al), vp(None)
    layer = sa.SaBlockLayer(*([al] * len(sa.BLOCK_LAYER_KEYS)))
    layers = (sa.SaBlockLayer * 2)(layer, layer)
    grads = (sa.SaBlockLayer * 2)(layer, layer)
    pr = _p(dtype=sa.SA_BF16, d=128, k=256)
    ws = lib.sa_block_workspace_size(ctypes.byref(pr), 2)
    assert ws > 0 and ws % 256 == 0
    assert lib.sa_block_workspace_size(ctypes.byref(pr), 9) == 0      # at most 8 layers
    pm = _p(mass_norm=True)
    assert lib.sa_block_workspace_size(ctypes.byref(pm), 2) == 0      # flags unsupported

    def fwd(pr=pr, L=2, off=ok, X=ok, P0=ok, lay=layers, out=ok, w=ok, wb=1 << 40):
        return lib.sa_block_forward(ctypes.byref(pr), L, off, X, P0, lay, out, w,
                                    ctypes.c_size_t(wb), nul)

    def bwd(pr=pr, L=2, off=ok, X=ok, P0=ok, lay=layers, dout=ok, dX=ok, dP0=ok, g=grads, w=ok,
            wb=1 << 40):
        return lib.sa_block_backward(ctypes.byref(pr), L, off, X, P0, lay, dout, dX, dP0, g, w,
                                     ctypes.c_size_t(wb), nul)

    assert fwd(L=0) == sa.SA_ERR_UNSUPPORTED
    assert fwd(L=9) == sa.SA_ERR_UNSUPPORTED
    assert fwd(pr=pm) == sa.SA_ERR_UNSUPPORTED
    assert fwd(pr=_p(k=0)) == sa.SA_ERR_BAD_SHAPE
    assert fwd(off=nul) == sa.SA_ERR_NULL_ARG
    assert fwd(out=nul) == sa.SA_ERR_NULL_ARG
    bad = (sa.SaBlockLayer * 2)(layer, layer)
    bad[1].W2 = None
    assert fwd(lay=bad) == sa.SA_ERR_NULL_ARG
    bad[1].W2 = al + 4
    assert fwd(lay=bad) == sa.SA_ERR_MISALIGNED
    assert fwd(X=vp(al + 8)) == sa.SA_ERR_MISALIGNED
    assert fwd(wb=256) == sa.SA_ERR_WORKSPACE_TOO_SMALL
    assert bwd(dout=nul) == sa.SA_ERR_NULL_ARG
    assert bwd(g=None) == sa.SA_ERR_NULL_ARG
    assert bwd(dX=nul) == sa.SA_ERR_NULL_ARG
    assert bwd(dP0=vp(al + 4)) == sa.SA_ERR_MISALIGNED
    assert bwd(wb=256) == sa.SA_ERR_WORKSPACE_TOO_SMALL


def test_action_fusion_argument_errors_are_synchronous():
    lib = sa.load()
    buf = ctypes.create_string_buffer(512)
    al = (ctypes.addressof(buf) + 255) & ~255
    vp = ctypes.c_void_p
    ok, nul = vp(al), vp(None)
    for dt in (sa.SA_F32, sa.SA_BF16):
        for op in (sa.SA_OP_FORWARD, sa.SA_OP_BACKWARD):
            assert lib.sa_action_fusion_workspace_size(128, dt, 1000, 8, op) > 0
    assert lib.sa_action_fusion_workspace_size(96, sa.SA_F32, 1000, 8, 0) == 0
    assert lib.sa_action_fusion_workspace_size(128, sa.SA_F32, 1000, 17, 0) == 0
    assert lib.sa_action_fusion_workspace_size(128, sa.SA_F32, 1000, 0, 0) == 0
    assert lib.sa_action_fusion_workspace_size(128, 7, 1000, 8, 0) == 0

    def fwd(d=128, dt=sa.SA_BF16, T=1000, nt=8, e=ok, types=ok, A=ok, W1=ok, W3=ok, W2=ok, x=ok,
            w=ok, wb=1 << 40):
        return lib.sa_action_fusion_forward(d, dt, T, nt, e, types, A, W1, W3, W2, x, w,
                                            ctypes.c_size_t(wb), nul)

    def bwd(e=ok, types=ok, dx=ok, de=ok, dA=ok, dW2=ok, wb=1 << 40):
        return lib.sa_action_fusion_backward(128, sa.SA_BF16, 1000, 8, e, types, ok, ok, ok, ok, dx,
                                             de, dA, ok, ok, dW2, ok, ctypes.c_size_t(wb), nul)

    assert fwd(dt=3) == sa.SA_ERR_BAD_DTYPE
    assert fwd(d=48) == sa.SA_ERR_BAD_SHAPE
    assert fwd(nt=17) == sa.SA_ERR_BAD_SHAPE
    assert fwd(W3=nul) == sa.SA_ERR_NULL_ARG
    assert fwd(types=nul) == sa.SA_ERR_NULL_ARG
    assert fwd(types=vp(al + 2)) == sa.SA_ERR_MISALIGNED
    assert fwd(W1=vp(al + 8)) == sa.SA_ERR_MISALIGNED
    assert fwd(wb=16) == sa.SA_ERR_WORKSPACE_TOO_SMALL
    assert bwd(dA=nul) == sa.SA_ERR_NULL_ARG
    assert bwd(de=nul) == sa.SA_ERR_NULL_ARG
    assert bwd(dW2=vp(al + 4)) == sa.SA_ERR_MISALIGNED
    assert bwd(dx=vp(al + 4)) == sa.SA_ERR_MISALIGNED
    assert bwd(wb=16) == sa.SA_ERR_WORKSPACE_TOO_SMALL


def test_stca_layer_argument_errors_are_synchronous():
    lib = sa.load()
    D, h, R = 512, 8, 7
    base = lib.sa_stca_workspace_size(D, h, R)
    a256 = lambda v: (v + 255) // 256 * 256
    want = a256(base) + 2 * a256(R * D * 4) + 3 * a256(R * 2 * D * 4)
    assert lib.sa_stca_layer_workspace_size(D, h, R) == want
    assert lib.sa_stca_layer_workspace_size(128, 4, R) == 0
    buf = ctypes.create_string_buffer(256)
    al = (ctypes.addressof(buf) + 15) & ~15
    vp = ctypes.c_void_p
    ok, nul = vp(al), vp(None)

    def call(D=256, h=4, R=3, Wo=ok, W1=ok, W3=ok, W2=ok, y=ok, o=nul, x_off=ok, ws=ok,
             ws_bytes=1 << 40):
        return lib.sa_stca_layer(2, D, h, 10, R, x_off, ok, ok, ok, ok, ok, ok, Wo, W1, W3, W2, y,
                                 o, nul, ws, ctypes.c_size_t(ws_bytes), nul)

    assert call(D=128) == sa.SA_ERR_BAD_SHAPE
    assert call(W1=nul) == sa.SA_ERR_NULL_ARG
    assert call(y=nul) == sa.SA_ERR_NULL_ARG
    assert call(x_off=nul) == sa.SA_ERR_NULL_ARG          # the attention's own checks
    assert call(W2=vp(al + 4)) == sa.SA_ERR_MISALIGNED
    assert call(o=vp(al + 8)) == sa.SA_ERR_MISALIGNED
    assert call(ws_bytes=16) == sa.SA_ERR_WORKSPACE_TOO_SMALL
    assert call(R=0, y=nul) == sa.SA_OK                   # nothing to compute
