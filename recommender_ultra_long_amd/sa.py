"""ctypes binding of libsa.so (include/sa.h).

Argument marshalling only: every step of Sketch Attention runs in the HIP
kernels of the library.  PyTorch provides device memory (outputs and the
workspace are torch tensors) and the stream (the current torch stream unless
one is given).  The library must have been built (``__graft_entry__.build()``
or ``python recommender_ultra_long_amd/build.py``); loading fails loudly
otherwise — there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

# SA_LIBRARY_PATH selects another build of the same library (the host-side
# AddressSanitizer build of the CPU checks).
_LIB_PATH = os.environ.get("SA_LIBRARY_PATH") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libsa.so")
_lib = None

SA_OK = 0
SA_ERR_NULL_ARG = 1
SA_ERR_BAD_SHAPE = 2
SA_ERR_BAD_DTYPE = 3
SA_ERR_UNSUPPORTED = 4
SA_ERR_WORKSPACE_TOO_SMALL = 5
SA_ERR_BAD_OFFSETS = 6
SA_ERR_MISALIGNED = 7
SA_ERR_HIP = 8
SA_ERR_DEVICE_TIMEOUT = 9

SA_F32 = 0
SA_BF16 = 1
SA_FLAG_MASS_NORM = 1
SA_FLAG_PER_USER_PROTOTYPES = 2
SA_FLAG_TOKEN_WISE = 4
SA_OP_FORWARD = 0
SA_OP_BACKWARD = 1

SA_PROFILE_MAX_KERNELS = 8

EXPORTED = ("sa_version", "sa_status_string", "sa_validate", "sa_workspace_size",
            "sa_forward", "sa_backward", "sa_forward_profiled", "sa_backward_profiled",
            "sa_get_device_status", "sa_fold_workspace_size", "sa_fold_prototypes",
            "sa_fold_prototypes_backward", "sa_block_workspace_size", "sa_block_forward",
            "sa_block_backward", "sa_action_fusion_workspace_size", "sa_action_fusion_forward",
            "sa_action_fusion_backward", "sa_stca_workspace_size", "sa_stca_attention",
            "sa_forward_noalloc", "sa_stca_layer_workspace_size", "sa_stca_layer")

# Bytes of the library's own workspace array used by sa_forward_noalloc.
SA_NOALLOC_SCRATCH_BYTES = 64 << 20

# Parameter names of one layer of the stacked block, in sa_block_layer order.
BLOCK_LAYER_KEYS = ("Wq", "Wk", "ln1_g", "ln1_b", "W1", "W3", "W2", "ln2_g", "ln2_b")


class SaProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("k", ctypes.c_int32), ("d", ctypes.c_int32),
                ("total_tokens", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("flags", ctypes.c_uint32)]


class SaBlockLayer(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in BLOCK_LAYER_KEYS]


class SaProfile(ctypes.Structure):
    _fields_ = [("events", ctypes.c_void_p * (2 * SA_PROFILE_MAX_KERNELS)),
                ("n_kernels", ctypes.c_int32),
                ("names", ctypes.c_char_p * SA_PROFILE_MAX_KERNELS)]


class SAError(RuntimeError):
    def __init__(self, status, where=""):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


def lib_path():
    return _LIB_PATH


def load():
    """Loads libsa.so once.  torch is imported first so that the library binds
    to the HIP runtime torch already loaded (same SONAME)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, sz, i32, i64p = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.POINTER(ctypes.c_int64)
    pp = ctypes.POINTER(SaProblem)
    lib.sa_version.restype = i32
    lib.sa_version.argtypes = []
    lib.sa_status_string.restype = ctypes.c_char_p
    lib.sa_status_string.argtypes = [i32]
    lib.sa_validate.restype = i32
    lib.sa_validate.argtypes = [pp, i64p]
    lib.sa_workspace_size.restype = sz
    lib.sa_workspace_size.argtypes = [pp, i32]
    lib.sa_forward.restype = i32
    lib.sa_forward.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sa_backward.restype = i32
    lib.sa_backward.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sa_forward_profiled.restype = i32
    lib.sa_forward_profiled.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                        ctypes.POINTER(SaProfile)]
    lib.sa_backward_profiled.restype = i32
    lib.sa_backward_profiled.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                         ctypes.POINTER(SaProfile)]
    lib.sa_get_device_status.restype = i32
    lib.sa_get_device_status.argtypes = [vp, vp]
    lib.sa_fold_workspace_size.restype = sz
    lib.sa_fold_workspace_size.argtypes = [i32, i32]
    lib.sa_fold_prototypes.restype = i32
    lib.sa_fold_prototypes.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp]
    lib.sa_fold_prototypes_backward.restype = i32
    lib.sa_fold_prototypes_backward.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                                sz, vp]
    lib.sa_block_workspace_size.restype = sz
    lib.sa_block_workspace_size.argtypes = [pp, i32]
    lib.sa_block_forward.restype = i32
    lib.sa_block_forward.argtypes = [pp, i32, vp, vp, vp, ctypes.POINTER(SaBlockLayer), vp, vp, sz,
                                     vp]
    lib.sa_block_backward.restype = i32
    lib.sa_block_backward.argtypes = [pp, i32, vp, vp, vp, ctypes.POINTER(SaBlockLayer), vp, vp, vp,
                                      ctypes.POINTER(SaBlockLayer), vp, sz, vp]
    i64 = ctypes.c_int64
    lib.sa_action_fusion_workspace_size.restype = sz
    lib.sa_action_fusion_workspace_size.argtypes = [i32, i32, i64, i32, i32]
    lib.sa_action_fusion_forward.restype = i32
    lib.sa_action_fusion_forward.argtypes = [i32, i32, i64, i32] + [vp] * 7 + [vp, sz, vp]
    lib.sa_action_fusion_backward.restype = i32
    lib.sa_action_fusion_backward.argtypes = [i32, i32, i64, i32] + [vp] * 12 + [vp, sz, vp]
    lib.sa_stca_workspace_size.restype = sz
    lib.sa_stca_workspace_size.argtypes = [i32, i32, i64]
    lib.sa_stca_attention.restype = i32
    lib.sa_stca_attention.argtypes = [i32, i32, i32, i64, i64] + [vp] * 9 + [vp, sz, vp]
    lib.sa_stca_layer_workspace_size.restype = sz
    lib.sa_stca_layer_workspace_size.argtypes = [i32, i32, i64]
    lib.sa_stca_layer.restype = i32
    lib.sa_stca_layer.argtypes = [i32, i32, i32, i64, i64] + [vp] * 14 + [vp, sz, vp]
    lib.sa_forward_noalloc.restype = i32
    lib.sa_forward_noalloc.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp]
    _lib = lib
    return lib


def version():
    return load().sa_version()


def status_string(status):
    return load().sa_status_string(int(status)).decode()


def make_problem(batch, k, d, total_tokens, dtype, mass_norm=False, per_user=False,
                 token_wise=False):
    if isinstance(dtype, torch.dtype):
        dtype = {torch.float32: SA_F32, torch.bfloat16: SA_BF16}.get(dtype, 99)
    flags = ((SA_FLAG_MASS_NORM if mass_norm else 0) | (SA_FLAG_PER_USER_PROTOTYPES if per_user else 0)
             | (SA_FLAG_TOKEN_WISE if token_wise else 0))
    return SaProblem(int(batch), int(k), int(d), int(total_tokens), int(dtype), flags)


def _tables(P, B):
    """(k, per_user) for a shared [k, d] table or a [B, k, d] stack."""
    if P.dim() == 2:
        return P.shape[0], False
    if P.dim() == 3 and P.shape[0] == B:
        return P.shape[1], True
    raise ValueError(f"P must be [k, d] or [{B}, k, d], got {tuple(P.shape)}")


def validate(problem, offsets_host=None):
    lib = load()
    ptr = None
    if offsets_host is not None:
        arr = np.ascontiguousarray(offsets_host, dtype=np.int64)
        ptr = arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    return lib.sa_validate(ctypes.byref(problem), ptr)


def workspace_size(problem, op=SA_OP_FORWARD):
    return int(load().sa_workspace_size(ctypes.byref(problem), int(op)))



# ---------------------------------------------------------------------------
# Argument checks.  Every public call checks its tensors before the first
# library call: the kernels take raw pointers and sizes, so a wrong dtype,
# shape or stride would otherwise be read as something else.  Mismatches raise
# ValueError; device placement is checked last, so that the dtype and shape
# checks also run on tensors that live on the host.

_FLOATS = (torch.float32, torch.bfloat16)


def _expect(name, t, dtype=None, shape=None, dtypes=None, optional=False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} must be one of {dtypes}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(int(v) for v in shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_device(device, **tensors):
    if device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU, got {device}")
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")


def _check_offsets_tensor(offsets):
    if isinstance(offsets, torch.Tensor):
        if offsets.dim() != 1 or offsets.numel() < 2:
            raise ValueError(f"offsets must be 1-D with at least 2 entries, got {tuple(offsets.shape)}")
        if offsets.dtype not in (torch.int64, torch.int32):
            raise ValueError(f"offsets must be an integer tensor, got {offsets.dtype}")
    else:
        arr = np.asarray(offsets)
        if arr.ndim != 1 or arr.size < 2 or not np.issubdtype(arr.dtype, np.integer):
            raise ValueError("offsets must be a 1-D integer array with at least 2 entries")


def _check_workspace(workspace, device):
    if workspace is not None:
        _expect("workspace", workspace, dtype=torch.uint8)
        _on_device(device, workspace=workspace)


def _check_sketch_args(offsets, X, P):
    """Shared checks of sa_forward / sa_backward: returns (B, T, d, k, per_user)."""
    _check_offsets_tensor(offsets)
    B = (offsets.numel() if isinstance(offsets, torch.Tensor) else len(offsets)) - 1
    _expect("X", X, dtypes=_FLOATS)
    if X.dim() != 2:
        raise ValueError(f"X must be [T, d], got {tuple(X.shape)}")
    _expect("P", P, dtype=X.dtype)
    T, d = X.shape
    if P.shape[-1] != d:
        raise ValueError(f"P's last dimension must equal X's width {d}, got {tuple(P.shape)}")
    k, per_user = _tables(P, B)
    return B, T, d, k, per_user

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _device_offsets(offsets, device):
    if isinstance(offsets, torch.Tensor):
        return offsets.to(device=device, dtype=torch.int64).contiguous()
    return torch.as_tensor(np.asarray(offsets, dtype=np.int64), device=device)


def _workspace(nbytes, device, workspace):
    if workspace is not None:
        return workspace
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


class KernelTimer:
    """Caller-owned events for the *_profiled entry points.  After a call and a
    synchronisation, times() returns [(kernel name, milliseconds)]."""

    def __init__(self):
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(2 * SA_PROFILE_MAX_KERNELS)]
        st = torch.cuda.current_stream()
        for e in self.events:          # torch creates the HIP event on first record
            e.record(st)
        torch.cuda.synchronize()
        self.prof = SaProfile()
        for i, e in enumerate(self.events):
            self.prof.events[i] = ctypes.c_void_p(e.cuda_event)

    def times(self):
        out = []
        for i in range(self.prof.n_kernels):
            name = self.prof.names[i].decode()
            out.append((name, self.events[2 * i].elapsed_time(self.events[2 * i + 1])))
        return out


def sa_forward(offsets, X, P, mass_norm=False, S=None, lse=None, mass=None, workspace=None,
               stream=None, want_lse=True, want_mass=True, timer=None):
    """Calls sa_forward.  offsets: int64 [B+1] (device tensor, or host array
    copied to X's device); X [T, d] and P float32 or bfloat16 on the GPU, P
    either [k, d] (shared) or [B, k, d] (one table per user).  Returns
    (S [B, k, d] f32, lse [T] f32 or None, mass [B, k] f32 or None)."""
    B, T, d, k, per_user = _check_sketch_args(offsets, X, P)
    _expect("S", S, torch.float32, (B, k, d), optional=True)
    _expect("lse", lse, torch.float32, (T,), optional=True)
    _expect("mass", mass, torch.float32, (B, k), optional=True)
    dev = P.device
    _check_workspace(workspace, dev)
    _on_device(dev, X=X, S=S, lse=lse, mass=mass)
    lib = load()
    off = _device_offsets(offsets, dev)
    pr = make_problem(B, k, d, T, X.dtype, mass_norm, per_user)
    if S is None:
        S = torch.empty((B, k, d), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((T,), dtype=torch.float32, device=dev)
    if mass is None and want_mass:
        mass = torch.empty((B, k), dtype=torch.float32, device=dev)
    ws_bytes = workspace_size(pr, SA_OP_FORWARD)
    ws = _workspace(ws_bytes, dev, workspace)
    args = (ctypes.byref(pr), _ptr(off), _ptr(X), _ptr(P), _ptr(S), _ptr(lse), _ptr(mass),
            _ptr(ws), ctypes.c_size_t(ws.numel() * ws.element_size()), _stream_handle(stream))
    if timer is None:
        st = lib.sa_forward(*args)
    else:
        st = lib.sa_forward_profiled(*args, ctypes.byref(timer.prof))
    if st != SA_OK:
        raise SAError(st, "sa_forward")
    return S, lse, mass


def sa_forward_noalloc(offsets, X, P, S, lse=None, mass=None, mass_norm=False, stream=None):
    """Calls sa_forward_noalloc: sa_forward with the library's own workspace
    array instead of a caller workspace.  Outputs are the caller's: S
    [B, k, d], and optionally lse [T] and mass [B, k] (float32, on the GPU).
    offsets must already be an int64 device tensor.  Returns (S, lse, mass)."""
    B, T, d, k, per_user = _check_sketch_args(offsets, X, P)
    _expect("S", S, torch.float32, (B, k, d))
    _expect("lse", lse, torch.float32, (T,), optional=True)
    _expect("mass", mass, torch.float32, (B, k), optional=True)
    if not isinstance(offsets, torch.Tensor) or offsets.dtype != torch.int64:
        raise ValueError("offsets must be an int64 device tensor")
    _expect("offsets", offsets)
    dev = P.device
    _on_device(dev, X=X, S=S, lse=lse, mass=mass, offsets=offsets)
    lib = load()
    pr = make_problem(B, k, d, T, X.dtype, mass_norm, per_user)
    st = lib.sa_forward_noalloc(ctypes.byref(pr), _ptr(offsets), _ptr(X), _ptr(P), _ptr(S),
                                _ptr(lse), _ptr(mass), _stream_handle(stream))
    if st != SA_OK:
        raise SAError(st, "sa_forward_noalloc")
    return S, lse, mass


def tokenwise_forward(offsets, X, P, S=None, lse=None, workspace=None, stream=None):
    """Calls sa_forward with SA_FLAG_TOKEN_WISE (the vanilla-attention baseline:
    softmax over each user's tokens).  Returns (S [B, k, d] f32, lse [B, k] f32)."""
    B, T, d, k, per_user = _check_sketch_args(offsets, X, P)
    if per_user:
        raise ValueError("the token-wise variant takes one shared [k, d] table")
    _expect("S", S, torch.float32, (B, k, d), optional=True)
    _expect("lse", lse, torch.float32, (B, k), optional=True)
    dev = P.device
    _check_workspace(workspace, dev)
    _on_device(dev, X=X, S=S, lse=lse)
    lib = load()
    off = _device_offsets(offsets, dev)
    pr = make_problem(B, k, d, T, X.dtype, token_wise=True)
    if S is None:
        S = torch.empty((B, k, d), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, k), dtype=torch.float32, device=dev)
    ws = _workspace(workspace_size(pr, SA_OP_FORWARD), dev, workspace)
    st = lib.sa_forward(ctypes.byref(pr), _ptr(off), _ptr(X), _ptr(P), _ptr(S), _ptr(lse), None,
                        _ptr(ws), ctypes.c_size_t(ws.numel() * ws.element_size()),
                        _stream_handle(stream))
    if st != SA_OK:
        raise SAError(st, "sa_forward (token-wise)")
    return S, lse


def tokenwise_backward(offsets, X, P, dS, S, lse, dX=None, dP=None, workspace=None, stream=None):
    """Calls sa_backward with SA_FLAG_TOKEN_WISE, given the token-wise
    forward's S [B, k, d] and lse [B, k].  Returns (dX [T, d], dP [k, d])."""
    B, T, d, k, per_user = _check_sketch_args(offsets, X, P)
    if per_user:
        raise ValueError("the token-wise variant takes one shared [k, d] table")
    _expect("dS", dS, torch.float32, (B, k, d))
    _expect("S", S, torch.float32, (B, k, d))
    _expect("lse", lse, torch.float32, (B, k))
    _expect("dX", dX, torch.float32, (T, d), optional=True)
    _expect("dP", dP, torch.float32, (k, d), optional=True)
    dev = P.device
    _check_workspace(workspace, dev)
    _on_device(dev, X=X, dS=dS, S=S, lse=lse, dX=dX, dP=dP)
    lib = load()
    off = _device_offsets(offsets, dev)
    pr = make_problem(B, k, d, T, X.dtype, token_wise=True)
    if dX is None:
        dX = torch.empty((T, d), dtype=torch.float32, device=dev)
    if dP is None:
        dP = torch.empty((k, d), dtype=torch.float32, device=dev)
    ws = _workspace(workspace_size(pr, SA_OP_BACKWARD), dev, workspace)
    st = lib.sa_backward(ctypes.byref(pr), _ptr(off), _ptr(X), _ptr(P), _ptr(dS), _ptr(lse), _ptr(S),
                         None, _ptr(dX), _ptr(dP), _ptr(ws),
                         ctypes.c_size_t(ws.numel() * ws.element_size()), _stream_handle(stream))
    if st != SA_OK:
        raise SAError(st, "sa_backward (token-wise)")
    return dX, dP


def sa_backward(offsets, X, P, dS, lse=None, S=None, mass=None, mass_norm=False, dX=None,
                dP=None, workspace=None, stream=None, timer=None):
    """Calls sa_backward.  Returns (dX [T, d] f32, dP f32 shaped like P:
    [k, d] summed over users, or [B, k, d] per user)."""
    B, T, d, k, per_user = _check_sketch_args(offsets, X, P)
    _expect("dS", dS, torch.float32, (B, k, d))
    _expect("lse", lse, torch.float32, (T,), optional=True)
    _expect("S", S, torch.float32, (B, k, d), optional=not mass_norm)
    _expect("mass", mass, torch.float32, (B, k), optional=not mass_norm)
    _expect("dX", dX, torch.float32, (T, d), optional=True)
    _expect("dP", dP, torch.float32, tuple(P.shape), optional=True)
    dev = P.device
    _check_workspace(workspace, dev)
    _on_device(dev, X=X, dS=dS, lse=lse, S=S, mass=mass, dX=dX, dP=dP)
    lib = load()
    off = _device_offsets(offsets, dev)
    pr = make_problem(B, k, d, T, X.dtype, mass_norm, per_user)
    if dX is None:
        dX = torch.empty((T, d), dtype=torch.float32, device=dev)
    if dP is None:
        dP = torch.empty(tuple(P.shape), dtype=torch.float32, device=dev)
    ws_bytes = workspace_size(pr, SA_OP_BACKWARD)
    ws = _workspace(ws_bytes, dev, workspace)
    args = (ctypes.byref(pr), _ptr(off), _ptr(X), _ptr(P), _ptr(dS), _ptr(lse), _ptr(S),
            _ptr(mass), _ptr(dX), _ptr(dP), _ptr(ws),
            ctypes.c_size_t(ws.numel() * ws.element_size()), _stream_handle(stream))
    if timer is None:
        st = lib.sa_backward(*args)
    else:
        st = lib.sa_backward_profiled(*args, ctypes.byref(timer.prof))
    if st != SA_OK:
        raise SAError(st, "sa_backward")
    return dX, dP


def _dtype_code(dtype):
    return {torch.float32: SA_F32, torch.bfloat16: SA_BF16}.get(dtype, 99)


def fold_prototypes(P, Wq, Wk, P_eff=None, stream=None):
    """Calls sa_fold_prototypes: P_eff = P W_Q W_K^T ([k, d], P's dtype), the
    prototype table whose affinities are Eq. (6)'s projected ones."""
    _expect("P", P, dtypes=_FLOATS)
    if P.dim() != 2:
        raise ValueError(f"P must be [k, d], got {tuple(P.shape)}")
    k, d = P.shape
    _expect("Wq", Wq, torch.float32, (d, d))
    _expect("Wk", Wk, torch.float32, (d, d))
    _expect("P_eff", P_eff, P.dtype, (k, d), optional=True)
    _on_device(P.device, Wq=Wq, Wk=Wk, P_eff=P_eff)
    lib = load()
    if P_eff is None:
        P_eff = torch.empty_like(P)
    st = lib.sa_fold_prototypes(int(k), int(d), _dtype_code(P.dtype), _ptr(P), _ptr(Wq), _ptr(Wk),
                                _ptr(P_eff), _stream_handle(stream))
    if st != SA_OK:
        raise SAError(st, "sa_fold_prototypes")
    return P_eff


def fold_prototypes_backward(P, Wq, Wk, dP_eff, workspace=None, stream=None):
    """Calls sa_fold_prototypes_backward.  Returns (dP [k, d], dW_Q [d, d],
    dW_K [d, d]), all float32."""
    _expect("P", P, dtypes=_FLOATS)
    if P.dim() != 2:
        raise ValueError(f"P must be [k, d], got {tuple(P.shape)}")
    k, d = P.shape
    _expect("Wq", Wq, torch.float32, (d, d))
    _expect("Wk", Wk, torch.float32, (d, d))
    _expect("dP_eff", dP_eff, torch.float32, (k, d))
    dev = P.device
    _check_workspace(workspace, dev)
    _on_device(dev, Wq=Wq, Wk=Wk, dP_eff=dP_eff)
    lib = load()
    dP = torch.empty((k, d), dtype=torch.float32, device=dev)
    dWq = torch.empty((d, d), dtype=torch.float32, device=dev)
    dWk = torch.empty((d, d), dtype=torch.float32, device=dev)
    ws_bytes = int(lib.sa_fold_workspace_size(int(k), int(d)))
    ws = _workspace(ws_bytes, dev, workspace)
    st = lib.sa_fold_prototypes_backward(int(k), int(d), _dtype_code(P.dtype), _ptr(P), _ptr(Wq),
                                         _ptr(Wk), _ptr(dP_eff), _ptr(dP), _ptr(dWq), _ptr(dWk),
                                         _ptr(ws), ctypes.c_size_t(ws.numel() * ws.element_size()),
                                         _stream_handle(stream))
    if st != SA_OK:
        raise SAError(st, "sa_fold_prototypes_backward")
    return dP, dWq, dWk


def _layer_shapes(d):
    return {"Wq": (d, d), "Wk": (d, d), "ln1_g": (d,), "ln1_b": (d,), "W1": (d, 2 * d),
            "W3": (d, 2 * d), "W2": (2 * d, d), "ln2_g": (d,), "ln2_b": (d,)}


def _check_layers(name, layers, d, device):
    shapes = _layer_shapes(d)
    for i, L in enumerate(layers):
        for key in BLOCK_LAYER_KEYS:
            t = L.get(key) if isinstance(L, dict) else None
            _expect(f"{name}[{i}]['{key}']", t, torch.float32, shapes[key])
    for L in layers:
        _on_device(device, **L)


def _layer_array(layers):
    """ctypes array of SaBlockLayer from a list of dicts of device tensors
    keyed by BLOCK_LAYER_KEYS (the same struct layout serves the gradients)."""
    arr = (SaBlockLayer * len(layers))()
    for i, L in enumerate(layers):
        for name in BLOCK_LAYER_KEYS:
            setattr(arr[i], name, _ptr(L[name]))
    return arr


def block_workspace(offsets_len, k, d, T, dtype, n_layers, device):
    pr = make_problem(offsets_len - 1, k, d, T, dtype)
    nbytes = int(load().sa_block_workspace_size(ctypes.byref(pr), int(n_layers)))
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def block_forward(offsets, X, P0, layers, out=None, workspace=None, stream=None):
    """Calls sa_block_forward: the stacked block (Eq. 12-16) over a CSR batch.
    X [T, d] (f32 or bf16), P0 [k, d] f32, layers: list of dicts of f32 device
    tensors keyed by BLOCK_LAYER_KEYS.  Returns (out [B, k, d] f32, workspace);
    pass the same workspace to block_backward."""
    _check_offsets_tensor(offsets)
    _expect("X", X, dtypes=_FLOATS)
    if X.dim() != 2:
        raise ValueError(f"X must be [T, d], got {tuple(X.shape)}")
    T, d = X.shape
    _expect("P0", P0, torch.float32)
    if P0.dim() != 2 or P0.shape[1] != d:
        raise ValueError(f"P0 must be [k, {d}], got {tuple(P0.shape)}")
    k = P0.shape[0]
    dev = P0.device
    _check_layers("layers", layers, d, dev)
    _on_device(dev, X=X)
    _check_workspace(workspace, dev)
    lib = load()
    off = _device_offsets(offsets, dev)
    B = off.numel() - 1
    _expect("out", out, torch.float32, (B, k, d), optional=True)
    _on_device(dev, out=out)
    pr = make_problem(B, k, d, T, X.dtype)
    if out is None:
        out = torch.empty((B, k, d), dtype=torch.float32, device=dev)
    ws = workspace if workspace is not None else block_workspace(B + 1, k, d, T, X.dtype,
                                                                 len(layers), dev)
    arr = _layer_array(layers)
    st = lib.sa_block_forward(ctypes.byref(pr), len(layers), _ptr(off), _ptr(X), _ptr(P0), arr,
                              _ptr(out), _ptr(ws), ctypes.c_size_t(ws.numel() * ws.element_size()),
                              _stream_handle(stream))
    if st != SA_OK:
        raise SAError(st, "sa_block_forward")
    return out, ws


def block_backward(offsets, X, P0, layers, dout, workspace, dX=None, dP0=None, grads=None,
                   stream=None):
    """Calls sa_block_backward with the workspace of the matching
    block_forward.  Returns (dX [T, d], dP0 [k, d], grads: list of dicts like
    layers), all f32."""
    _check_offsets_tensor(offsets)
    _expect("X", X, dtypes=_FLOATS)
    if X.dim() != 2:
        raise ValueError(f"X must be [T, d], got {tuple(X.shape)}")
    T, d = X.shape
    _expect("P0", P0, torch.float32)
    if P0.dim() != 2 or P0.shape[1] != d:
        raise ValueError(f"P0 must be [k, {d}], got {tuple(P0.shape)}")
    k = P0.shape[0]
    dev = P0.device
    _check_layers("layers", layers, d, dev)
    _on_device(dev, X=X)
    if grads is not None:
        _check_layers("grads", grads, d, dev)
    _expect("workspace", workspace, torch.uint8)
    _on_device(dev, workspace=workspace)
    lib = load()
    off = _device_offsets(offsets, dev)
    B = off.numel() - 1
    _expect("dout", dout, torch.float32, (B, k, d))
    _expect("dX", dX, torch.float32, (T, d), optional=True)
    _expect("dP0", dP0, torch.float32, (k, d), optional=True)
    _on_device(dev, dout=dout, dX=dX, dP0=dP0)
    pr = make_problem(B, k, d, T, X.dtype)
    if dX is None:
        dX = torch.empty((T, d), dtype=torch.float32, device=dev)
    if dP0 is None:
        dP0 = torch.empty((k, d), dtype=torch.float32, device=dev)
    if grads is None:
        grads = [{name: torch.empty_like(L[name]) for name in BLOCK_LAYER_KEYS} for L in layers]
    st = lib.sa_block_backward(ctypes.byref(pr), len(layers), _ptr(off), _ptr(X), _ptr(P0),
                               _layer_array(layers), _ptr(dout), _ptr(dX), _ptr(dP0),
                               _layer_array(grads), _ptr(workspace),
                               ctypes.c_size_t(workspace.numel() * workspace.element_size()),
                               _stream_handle(stream))
    if st != SA_OK:
        raise SAError(st, "sa_block_backward")
    return dX, dP0, grads


def _action_ws(d, dtype, T, n_types, op, device, workspace):
    n = int(load().sa_action_fusion_workspace_size(int(d), _dtype_code(dtype), int(T), int(n_types),
                                                   int(op)))
    return _workspace(n, device, workspace)


def _check_action_args(e, types, A, W1, W3, W2, workspace):
    _expect("e", e, dtypes=_FLOATS)
    if e.dim() != 2:
        raise ValueError(f"e must be [T, d], got {tuple(e.shape)}")
    T, d = e.shape
    _expect("types", types, torch.int32, (T,))
    _expect("A", A, torch.float32)
    if A.dim() != 2 or A.shape[1] != d:
        raise ValueError(f"A must be [n_types, {d}], got {tuple(A.shape)}")
    _expect("W1", W1, torch.float32, (2 * d, 2 * d))
    _expect("W3", W3, torch.float32, (2 * d, 2 * d))
    _expect("W2", W2, torch.float32, (2 * d, d))
    _on_device(e.device, types=types, A=A, W1=W1, W3=W3, W2=W2)
    _check_workspace(workspace, e.device)
    return T, d, A.shape[0]


def action_fusion_forward(e, types, A, W1, W3, W2, x=None, workspace=None, stream=None):
    """Calls sa_action_fusion_forward: x = e + SwiGLU([e; A[types]]) (Eq. 20).
    e [T, d] f32 or bf16, types int32 [T], A [n_types, d], W1, W3 [2d, 2d],
    W2 [2d, d] f32.  Returns x [T, d] in e's dtype."""
    T, d, n_types = _check_action_args(e, types, A, W1, W3, W2, workspace)
    _expect("x", x, e.dtype, (T, d), optional=True)
    _on_device(e.device, x=x)
    lib = load()
    if x is None:
        x = torch.empty_like(e)
    ws = _action_ws(d, e.dtype, T, n_types, SA_OP_FORWARD, e.device, workspace)
    st = lib.sa_action_fusion_forward(int(d), _dtype_code(e.dtype), int(T), int(n_types), _ptr(e),
                                      _ptr(types), _ptr(A), _ptr(W1), _ptr(W3), _ptr(W2), _ptr(x),
                                      _ptr(ws), ctypes.c_size_t(ws.numel() * ws.element_size()),
                                      _stream_handle(stream))
    if st != SA_OK:
        raise SAError(st, "sa_action_fusion_forward")
    return x


def action_fusion_backward(e, types, A, W1, W3, W2, dx, workspace=None, stream=None):
    """Calls sa_action_fusion_backward.  Returns (de [T, d], dA, dW1, dW3,
    dW2), all f32."""
    T, d, n_types = _check_action_args(e, types, A, W1, W3, W2, workspace)
    _expect("dx", dx, torch.float32, (T, d))
    _on_device(e.device, dx=dx)
    lib = load()
    dev = e.device
    de = torch.empty((T, d), dtype=torch.float32, device=dev)
    dA, dW1, dW3, dW2 = (torch.empty_like(t) for t in (A, W1, W3, W2))
    ws = _action_ws(d, e.dtype, T, n_types, SA_OP_BACKWARD, dev, workspace)
    st = lib.sa_action_fusion_backward(int(d), _dtype_code(e.dtype), int(T), int(n_types), _ptr(e),
                                       _ptr(types), _ptr(A), _ptr(W1), _ptr(W3), _ptr(W2),
                                       _ptr(dx), _ptr(de), _ptr(dA), _ptr(dW1), _ptr(dW3),
                                       _ptr(dW2), _ptr(ws),
                                       ctypes.c_size_t(ws.numel() * ws.element_size()),
                                       _stream_handle(stream))
    if st != SA_OK:
        raise SAError(st, "sa_action_fusion_backward")
    return de, dA, dW1, dW3, dW2


def stca_attention(x_off, X, t_off, Q, Wq, Wk, Wv, h, o=None, lse=None, workspace=None,
                   stream=None):
    """Calls sa_stca_attention (Eq. 24): per target and head, softmax over the
    target's user's rows of X.  x_off, t_off: int64 [B+1] (device); X bf16
    [L, D]; Q, Wq, Wk, Wv f32.  Returns (o [R, D], lse [R, h])."""
    _check_offsets_tensor(x_off)
    _check_offsets_tensor(t_off)
    _expect("X", X, torch.bfloat16)
    if X.dim() != 2:
        raise ValueError(f"X must be [L, D], got {tuple(X.shape)}")
    D = X.shape[1]
    _expect("Q", Q, torch.float32)
    if Q.dim() != 2 or Q.shape[1] != D:
        raise ValueError(f"Q must be [R, {D}], got {tuple(Q.shape)}")
    for name, w in (("Wq", Wq), ("Wk", Wk), ("Wv", Wv)):
        _expect(name, w, torch.float32, (D, D))
    _expect("o", o, torch.float32, (Q.shape[0], D), optional=True)
    _expect("lse", lse, torch.float32, (Q.shape[0], int(h)), optional=True)
    dev = Q.device
    _check_workspace(workspace, dev)
    _on_device(dev, X=X, Wq=Wq, Wk=Wk, Wv=Wv, o=o, lse=lse)
    lib = load()
    xo = _device_offsets(x_off, dev)
    to = _device_offsets(t_off, dev)
    B = xo.numel() - 1
    L, D = X.shape
    R = Q.shape[0]
    if o is None:
        o = torch.empty((R, D), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((R, h), dtype=torch.float32, device=dev)
    n = int(lib.sa_stca_workspace_size(int(D), int(h), int(R)))
    ws = _workspace(n, dev, workspace)
    st = lib.sa_stca_attention(int(B), int(D), int(h), int(L), int(R), _ptr(xo), _ptr(to), _ptr(X),
                               _ptr(Q), _ptr(Wq), _ptr(Wk), _ptr(Wv), _ptr(o), _ptr(lse), _ptr(ws),
                               ctypes.c_size_t(ws.numel() * ws.element_size()),
                               _stream_handle(stream))
    if st != SA_OK:
        raise SAError(st, "sa_stca_attention")
    return o, lse


def stca_layer(x_off, X, t_off, Q, Wq, Wk, Wv, Wo, W1, W3, W2, h, y=None, o=None, lse=None,
               workspace=None, stream=None):
    """Calls sa_stca_layer (Eq. 26): the attention of stca_attention, then
    a = q + o W_O and y = a + SwiGLU(a) with hidden width 2D.  Wo [D, D],
    W1, W3 [D, 2D], W2 [2D, D] f32.  Returns (y [R, D], o [R, D], lse [R, h])."""
    _check_offsets_tensor(x_off)
    _check_offsets_tensor(t_off)
    _expect("X", X, torch.bfloat16)
    if X.dim() != 2:
        raise ValueError(f"X must be [L, D], got {tuple(X.shape)}")
    D = X.shape[1]
    _expect("Q", Q, torch.float32)
    if Q.dim() != 2 or Q.shape[1] != D:
        raise ValueError(f"Q must be [R, {D}], got {tuple(Q.shape)}")
    R = Q.shape[0]
    for name, w, shape in (("Wq", Wq, (D, D)), ("Wk", Wk, (D, D)), ("Wv", Wv, (D, D)),
                           ("Wo", Wo, (D, D)), ("W1", W1, (D, 2 * D)), ("W3", W3, (D, 2 * D)),
                           ("W2", W2, (2 * D, D))):
        _expect(name, w, torch.float32, shape)
    _expect("y", y, torch.float32, (R, D), optional=True)
    _expect("o", o, torch.float32, (R, D), optional=True)
    _expect("lse", lse, torch.float32, (R, int(h)), optional=True)
    dev = Q.device
    _check_workspace(workspace, dev)
    _on_device(dev, X=X, Wq=Wq, Wk=Wk, Wv=Wv, Wo=Wo, W1=W1, W3=W3, W2=W2, y=y, o=o, lse=lse)
    lib = load()
    xo = _device_offsets(x_off, dev)
    to = _device_offsets(t_off, dev)
    B = xo.numel() - 1
    L = X.shape[0]
    if y is None:
        y = torch.empty((R, D), dtype=torch.float32, device=dev)
    if o is None:
        o = torch.empty((R, D), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((R, h), dtype=torch.float32, device=dev)
    n = int(lib.sa_stca_layer_workspace_size(int(D), int(h), int(R)))
    ws = _workspace(n, dev, workspace)
    st = lib.sa_stca_layer(int(B), int(D), int(h), int(L), int(R), _ptr(xo), _ptr(to), _ptr(X),
                           _ptr(Q), _ptr(Wq), _ptr(Wk), _ptr(Wv), _ptr(Wo), _ptr(W1), _ptr(W3),
                           _ptr(W2), _ptr(y), _ptr(o), _ptr(lse), _ptr(ws),
                           ctypes.c_size_t(ws.numel() * ws.element_size()), _stream_handle(stream))
    if st != SA_OK:
        raise SAError(st, "sa_stca_layer")
    return y, o, lse


def sa_get_device_status(workspace, stream=None):
    return load().sa_get_device_status(_ptr(workspace), _stream_handle(stream))


class SketchAttention(torch.autograd.Function):
    """Autograd wrapper: S = SA(X, P) over a CSR-ragged batch.  Gradients flow
    to X and P through sa_backward."""

    @staticmethod
    def forward(ctx, X, P, offsets, mass_norm=False):
        off = _device_offsets(offsets, P.device)
        S, lse, mass = sa_forward(off, X, P, mass_norm)
        ctx.save_for_backward(X, P, off, S, lse, mass)
        ctx.mass_norm = mass_norm
        return S

    @staticmethod
    def backward(ctx, dS):
        X, P, off, S, lse, mass = ctx.saved_tensors
        dX, dP = sa_backward(off, X, P, dS.contiguous().float(), lse, S, mass, ctx.mass_norm)
        return dX.to(X.dtype), dP.to(P.dtype), None, None
