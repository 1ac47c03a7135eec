"""mLSTM matrix-memory cell forward pass on MI355X (gfx950).

Thin Python binding over the C ABI of ``libmlstm.so`` (declared in
``include/mlstm.h``).  The functions keep the C names.  They only check and
marshal arguments: torch supplies device memory and the current stream, and
every step of the computation runs in the library's HIP kernels.  There is no
fallback: if the library is missing or a call fails, an exception is raised.

    h, (C1, n1, m1) = mlstm_fwd_chunkwise(q, k, v, i_pre, f_pre, o_pre,
                                          C0, n0, m0, chunk=64)
    h, (C1, n1, m1) = mlstm_fwd_parallel(q, k, v, i_pre, f_pre, o_pre, C0, n0, m0)
    h, (C, n, m)    = mlstm_step(q, k, v, i_pre, f_pre, o_pre, C, n, m)
    y               = mlstm_groupnorm_ogate(h, o_pre, gamma, beta, eps=1e-5)
    y, state        = mlstm_causal_conv1d(x, w, bias, state)
    h, (c, n, m, h1) = mlstm_slstm_fwd(wx, R, c0, n0, m0, h0)     # sLSTM cell

Shapes: q, k [B,H,T,d_qk]; v, o_pre, h [B,H,T,d_v]; i_pre, f_pre [B,H,T];
C [B,H,d_qk,d_v]; n [B,H,d_qk]; m [B,H] (the step drops T).  q, k, v are
float32 or bfloat16 (h gets the same dtype); o_pre is float32 or bfloat16 or
None; gates and state are float32.  k is expected pre-scaled by 1/sqrt(d_qk).
"""
from __future__ import annotations

import contextlib
import ctypes
import functools
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "mlstm_fwd_chunkwise", "mlstm_fwd_chunkwise_noalloc", "mlstm_fwd_parallel", "mlstm_step",
    "mlstm_bwd_chunkwise",
    "mlstm_bwd_chunkwise_workspace_bytes", "mlstm_groupnorm_ogate", "mlstm_causal_conv1d",
    "mlstm_slstm_fwd", "SlstmProblem",
    "mlstm_fwd_chunkwise_workspace_bytes", "mlstm_fwd_parallel_workspace_bytes",
    "mlstm_version", "library_path", "load_library", "MLSTMError",
    "MLSTM_OK", "MLSTM_ERR_INVALID_ARG", "MLSTM_ERR_UNSUPPORTED", "MLSTM_ERR_DEVICE",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libmlstm.so")

MLSTM_OK = 0
MLSTM_ERR_INVALID_ARG = 1
MLSTM_ERR_UNSUPPORTED = 2
MLSTM_ERR_DEVICE = 3
MLSTM_F32 = 0
MLSTM_BF16 = 1
MLSTM_FGATE_SIGMOID = 0
MLSTM_FGATE_EXP = 1


class MLSTMError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"mlstm status {status}: {detail}")
        self.status = status
        self.detail = detail


class Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("T", ctypes.c_int64),
                ("d_qk", ctypes.c_int64), ("d_v", ctypes.c_int64),
                ("qkv_dtype", ctypes.c_int32), ("o_dtype", ctypes.c_int32),
                ("fgate", ctypes.c_int32), ("reserved", ctypes.c_int32)]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libmlstm.so (built in-tree by ``build.build()``); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build() "
                           "(or python mlstm_matrix_memory_chunkwise_amd/build.py)")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    PP = ctypes.POINTER(Problem)
    seq = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.mlstm_fwd_chunkwise.argtypes = [PP, i64] + seq
    lib.mlstm_fwd_chunkwise.restype = ctypes.c_int
    lib.mlstm_fwd_chunkwise_noalloc.argtypes = [PP, i64] + [vp] * 13 + [vp]
    lib.mlstm_fwd_chunkwise_noalloc.restype = ctypes.c_int
    lib.mlstm_fwd_parallel.argtypes = [PP] + seq
    lib.mlstm_fwd_parallel.restype = ctypes.c_int
    lib.mlstm_step.argtypes = [PP] + [vp] * 14
    lib.mlstm_step.restype = ctypes.c_int
    lib.mlstm_fwd_chunkwise_workspace_bytes.argtypes = [PP, i64, ctypes.POINTER(sz)]
    lib.mlstm_fwd_chunkwise_workspace_bytes.restype = ctypes.c_int
    lib.mlstm_fwd_parallel_workspace_bytes.argtypes = [PP, ctypes.POINTER(sz)]
    lib.mlstm_fwd_parallel_workspace_bytes.restype = ctypes.c_int
    lib.mlstm_bwd_chunkwise.argtypes = [PP, i64] + [vp] * 23 + [sz, vp]
    lib.mlstm_bwd_chunkwise.restype = ctypes.c_int
    lib.mlstm_bwd_chunkwise_workspace_bytes.argtypes = [PP, i64, ctypes.POINTER(sz)]
    lib.mlstm_bwd_chunkwise_workspace_bytes.restype = ctypes.c_int
    lib.mlstm_groupnorm_ogate.argtypes = [i64, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                          vp, vp, vp, vp, ctypes.c_float, vp, vp]
    lib.mlstm_groupnorm_ogate.restype = ctypes.c_int
    lib.mlstm_causal_conv1d.argtypes = [i64, i64, i64, i64, ctypes.c_int, vp, vp, vp, vp, vp,
                                        vp, vp]
    lib.mlstm_causal_conv1d.restype = ctypes.c_int
    lib.mlstm_slstm_fwd.argtypes = [ctypes.POINTER(SlstmProblem)] + [vp] * 12
    lib.mlstm_slstm_fwd.restype = ctypes.c_int
    lib.mlstm_status_string.argtypes = [ctypes.c_int]
    lib.mlstm_status_string.restype = ctypes.c_char_p
    lib.mlstm_last_error_detail.argtypes = []
    lib.mlstm_last_error_detail.restype = ctypes.c_char_p
    lib.mlstm_version.argtypes = []
    lib.mlstm_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def mlstm_version() -> str:
    return load_library().mlstm_version().decode()


def _check(status: int):
    if status != MLSTM_OK:
        lib = load_library()
        raise MLSTMError(status, lib.mlstm_last_error_detail().decode())


_DT = {torch.float32: MLSTM_F32, torch.bfloat16: MLSTM_BF16}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev_tensor(name, t, dtype=None, shape=None, device=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _fgate(fgate) -> int:
    if fgate in ("sigmoid", MLSTM_FGATE_SIGMOID):
        return MLSTM_FGATE_SIGMOID
    if fgate in ("exp", MLSTM_FGATE_EXP):
        return MLSTM_FGATE_EXP
    raise ValueError(f"unknown forget gate {fgate!r}")


def _stream_handle(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on_stream(stream):
    """Context in which a call allocates its outputs and scratch: the stream
    the kernels are enqueued on.  torch's caching allocator then hands a freed
    block (the workspace, released on return) only to work ordered after
    these kernels on that stream, never to another stream while they still
    use it."""
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _allocates_on_stream(fn):
    """Runs an entry point (keyword argument ``stream``) under _on_stream."""
    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        with _on_stream(kwargs.get("stream")):
            return fn(*args, **kwargs)
    return wrapper


def _seq_problem(q, k, v, i_pre, f_pre, o_pre, C0, n0, m0, fgate):
    q = _dev_tensor("q", q, (torch.float32, torch.bfloat16))
    if q.dim() != 4:
        raise ValueError("q must be [B,H,T,d_qk]")
    B, H, T, dqk = q.shape
    dev = q.device
    k = _dev_tensor("k", k, q.dtype, (B, H, T, dqk), dev)
    v = _dev_tensor("v", v, q.dtype, None, dev)
    if v.dim() != 4 or tuple(v.shape[:3]) != (B, H, T):
        raise ValueError("v must be [B,H,T,d_v]")
    dv = v.shape[3]
    i_pre = _dev_tensor("i_pre", i_pre, torch.float32, (B, H, T), dev)
    f_pre = _dev_tensor("f_pre", f_pre, torch.float32, (B, H, T), dev)
    o_pre = _dev_tensor("o_pre", o_pre, (torch.float32, torch.bfloat16), (B, H, T, dv), dev)
    C0 = _dev_tensor("C0", C0, torch.float32, (B, H, dqk, dv), dev)
    n0 = _dev_tensor("n0", n0, torch.float32, (B, H, dqk), dev)
    m0 = _dev_tensor("m0", m0, torch.float32, (B, H), dev)
    p = Problem(B, H, T, dqk, dv, _DT[q.dtype],
                _DT[o_pre.dtype] if o_pre is not None else MLSTM_F32, _fgate(fgate), 0)
    return p, (q, k, v, i_pre, f_pre, o_pre, C0, n0, m0)


def _outputs(p, q, out, return_state, state_out=None):
    B, H, T, dqk, dv = p.B, p.H, p.T, p.d_qk, p.d_v
    dev = q.device
    if out is not None:
        h = _dev_tensor("out", out, q.dtype, (B, H, T, dv), dev)
    else:
        h = torch.empty((B, H, T, dv), dtype=q.dtype, device=dev)
    if state_out is not None:
        if not return_state:
            raise ValueError("state_out is given but return_state is False")
        C1 = _dev_tensor("C1", state_out[0], torch.float32, (B, H, dqk, dv), dev)
        n1 = _dev_tensor("n1", state_out[1], torch.float32, (B, H, dqk), dev)
        m1 = _dev_tensor("m1", state_out[2], torch.float32, (B, H), dev)
    elif return_state:
        C1 = torch.empty((B, H, dqk, dv), dtype=torch.float32, device=dev)
        n1 = torch.empty((B, H, dqk), dtype=torch.float32, device=dev)
        m1 = torch.empty((B, H), dtype=torch.float32, device=dev)
    else:
        C1 = n1 = m1 = None
    return h, C1, n1, m1


def mlstm_fwd_chunkwise_workspace_bytes(p: Problem, chunk: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().mlstm_fwd_chunkwise_workspace_bytes(ctypes.byref(p), int(chunk),
                                                              ctypes.byref(n)))
    return int(n.value)


def mlstm_fwd_parallel_workspace_bytes(p: Problem) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().mlstm_fwd_parallel_workspace_bytes(ctypes.byref(p), ctypes.byref(n)))
    return int(n.value)


@_allocates_on_stream
def mlstm_fwd_chunkwise(q, k, v, i_pre, f_pre, o_pre=None, C0=None, n0=None, m0=None, *,
                        chunk: int = 64, fgate="sigmoid", return_state: bool = True,
                        out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                        state_out=None, stream=None):
    """Chunkwise forward pass.  Returns (h, (C1, n1, m1)) or (h, None).
    ``state_out`` = (C1, n1, m1) tensors to write the final state into."""
    lib = load_library()
    p, (q, k, v, i_pre, f_pre, o_pre, C0, n0, m0) = _seq_problem(
        q, k, v, i_pre, f_pre, o_pre, C0, n0, m0, fgate)
    h, C1, n1, m1 = _outputs(p, q, out, return_state, state_out)
    need = mlstm_fwd_chunkwise_workspace_bytes(p, chunk)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.mlstm_fwd_chunkwise(ctypes.byref(p), int(chunk), _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(i_pre), _ptr(f_pre), _ptr(o_pre), _ptr(C0), _ptr(n0),
                                   _ptr(m0), _ptr(h), _ptr(C1), _ptr(n1), _ptr(m1),
                                   _ptr(workspace), wbytes, _stream_handle(stream)))
    return h, ((C1, n1, m1) if return_state else None)


def mlstm_fwd_chunkwise_noalloc(q, k, v, i_pre, f_pre, o_pre=None, C0=None, n0=None, m0=None, *,
                                out, state_out=None, chunk: int = 64, fgate="sigmoid",
                                stream=None):
    """mlstm_fwd_chunkwise through the entry point that allocates nothing (its
    scratch is a fixed device array of the library).  The caller passes every
    output: ``out`` (h) and optionally ``state_out`` = (C1, n1, m1).  Returns
    (h, (C1, n1, m1)) or (h, None)."""
    lib = load_library()
    p, (q, k, v, i_pre, f_pre, o_pre, C0, n0, m0) = _seq_problem(
        q, k, v, i_pre, f_pre, o_pre, C0, n0, m0, fgate)
    if out is None:
        raise ValueError("out is required (this entry point allocates nothing)")
    h, C1, n1, m1 = _outputs(p, q, out, state_out is not None, state_out)
    _check(lib.mlstm_fwd_chunkwise_noalloc(ctypes.byref(p), int(chunk), _ptr(q), _ptr(k), _ptr(v),
                                           _ptr(i_pre), _ptr(f_pre), _ptr(o_pre), _ptr(C0),
                                           _ptr(n0), _ptr(m0), _ptr(h), _ptr(C1), _ptr(n1),
                                           _ptr(m1), _stream_handle(stream)))
    return h, ((C1, n1, m1) if state_out is not None else None)


@_allocates_on_stream
def mlstm_fwd_parallel(q, k, v, i_pre, f_pre, o_pre=None, C0=None, n0=None, m0=None, *,
                       fgate="sigmoid", return_state: bool = True,
                       out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                       state_out=None, stream=None):
    """Parallel (quadratic) forward pass.  Returns (h, (C1, n1, m1)) or (h, None).
    ``state_out`` = (C1, n1, m1) tensors to write the final state into."""
    lib = load_library()
    p, (q, k, v, i_pre, f_pre, o_pre, C0, n0, m0) = _seq_problem(
        q, k, v, i_pre, f_pre, o_pre, C0, n0, m0, fgate)
    h, C1, n1, m1 = _outputs(p, q, out, return_state, state_out)
    need = mlstm_fwd_parallel_workspace_bytes(p)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check(lib.mlstm_fwd_parallel(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(i_pre),
                                  _ptr(f_pre), _ptr(o_pre), _ptr(C0), _ptr(n0), _ptr(m0),
                                  _ptr(h), _ptr(C1), _ptr(n1), _ptr(m1), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(),
                                  _stream_handle(stream)))
    return h, ((C1, n1, m1) if return_state else None)


def mlstm_bwd_chunkwise_workspace_bytes(p: Problem, chunk: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().mlstm_bwd_chunkwise_workspace_bytes(ctypes.byref(p), int(chunk),
                                                              ctypes.byref(n)))
    return int(n.value)


@_allocates_on_stream
def mlstm_bwd_chunkwise(q, k, v, i_pre, f_pre, o_pre, C0, n0, m0, h, dh, dC1=None, dn1=None, *,
                        chunk: int = 32, fgate="sigmoid", workspace: Optional[torch.Tensor] = None,
                        stream=None):
    """Chunkwise backward pass (see mlstm_bwd_chunkwise in include/mlstm.h).

    h is the forward output of the same inputs; dh its gradient (same dtype);
    dC1, dn1 the gradient of the final memory in the stored final scale, or
    None.  Returns a dict of float32 tensors dq, dk, dv, di, df, do (None
    without o_pre), dC0, dn0, dm0.
    """
    lib = load_library()
    p, (q, k, v, i_pre, f_pre, o_pre, C0, n0, m0) = _seq_problem(
        q, k, v, i_pre, f_pre, o_pre, C0, n0, m0, fgate)
    B, H, T, dqk, dv = p.B, p.H, p.T, p.d_qk, p.d_v
    dev = q.device
    h = _dev_tensor("h", h, q.dtype, (B, H, T, dv), dev)
    dh = _dev_tensor("dh", dh, q.dtype, (B, H, T, dv), dev)
    dC1 = _dev_tensor("dC1", dC1, torch.float32, (B, H, dqk, dv), dev)
    dn1 = _dev_tensor("dn1", dn1, torch.float32, (B, H, dqk), dev)
    f32 = dict(dtype=torch.float32, device=dev)
    g = dict(dq=torch.empty((B, H, T, dqk), **f32), dk=torch.empty((B, H, T, dqk), **f32),
             dv=torch.empty((B, H, T, dv), **f32), di=torch.empty((B, H, T), **f32),
             df=torch.empty((B, H, T), **f32),
             do=None if o_pre is None else torch.empty((B, H, T, dv), **f32),
             dC0=torch.empty((B, H, dqk, dv), **f32), dn0=torch.empty((B, H, dqk), **f32),
             dm0=torch.empty((B, H), **f32))
    need = mlstm_bwd_chunkwise_workspace_bytes(p, chunk)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _check(lib.mlstm_bwd_chunkwise(ctypes.byref(p), int(chunk), _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(i_pre), _ptr(f_pre), _ptr(o_pre), _ptr(C0), _ptr(n0),
                                   _ptr(m0), _ptr(h), _ptr(dh), _ptr(dC1), _ptr(dn1),
                                   _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["di"]),
                                   _ptr(g["df"]), _ptr(g["do"]), _ptr(g["dC0"]), _ptr(g["dn0"]),
                                   _ptr(g["dm0"]), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(),
                                   _stream_handle(stream)))
    return g


@_allocates_on_stream
def mlstm_step(q, k, v, i_pre, f_pre, o_pre, C, n, m, *, fgate="sigmoid",
               inplace: bool = False, out: Optional[torch.Tensor] = None,
               state_out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
               stream=None):
    """One decode step.  Returns (h, (C', n', m')).  With inplace=True the state
    tensors C, n, m are updated in place and returned."""
    lib = load_library()
    q = _dev_tensor("q", q, (torch.float32, torch.bfloat16))
    if q.dim() != 3:
        raise ValueError("q must be [B,H,d_qk]")
    B, H, dqk = q.shape
    dev = q.device
    k = _dev_tensor("k", k, q.dtype, (B, H, dqk), dev)
    v = _dev_tensor("v", v, q.dtype, None, dev)
    if v.dim() != 3 or tuple(v.shape[:2]) != (B, H):
        raise ValueError("v must be [B,H,d_v]")
    dv = v.shape[2]
    i_pre = _dev_tensor("i_pre", i_pre, torch.float32, (B, H), dev)
    f_pre = _dev_tensor("f_pre", f_pre, torch.float32, (B, H), dev)
    o_pre = _dev_tensor("o_pre", o_pre, (torch.float32, torch.bfloat16), (B, H, dv), dev)
    C = _dev_tensor("C", C, torch.float32, (B, H, dqk, dv), dev)
    n = _dev_tensor("n", n, torch.float32, (B, H, dqk), dev)
    m = _dev_tensor("m", m, torch.float32, (B, H), dev)
    if inplace:
        C1, n1, m1 = C, n, m
    elif state_out is not None:
        C1 = _dev_tensor("C_out", state_out[0], torch.float32, (B, H, dqk, dv), dev)
        n1 = _dev_tensor("n_out", state_out[1], torch.float32, (B, H, dqk), dev)
        m1 = _dev_tensor("m_out", state_out[2], torch.float32, (B, H), dev)
    else:
        C1, n1, m1 = torch.empty_like(C), torch.empty_like(n), torch.empty_like(m)
    h = (_dev_tensor("out", out, q.dtype, (B, H, dv), dev) if out is not None
         else torch.empty((B, H, dv), dtype=q.dtype, device=dev))
    p = Problem(B, H, 1, dqk, dv, _DT[q.dtype],
                _DT[o_pre.dtype] if o_pre is not None else MLSTM_F32, _fgate(fgate), 0)
    _check(lib.mlstm_step(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(i_pre), _ptr(f_pre),
                          _ptr(o_pre), _ptr(C), _ptr(n), _ptr(m), _ptr(C1), _ptr(n1), _ptr(m1),
                          _ptr(h), _stream_handle(stream)))
    return h, (C1, n1, m1)


@_allocates_on_stream
def mlstm_groupnorm_ogate(h, o_pre=None, gamma=None, beta=None, eps: float = 1e-5, *,
                          out: Optional[torch.Tensor] = None, stream=None):
    """Per-head group normalization of the cell output with the output gate
    (see mlstm_groupnorm_ogate in include/mlstm.h).  h [B,H,T,d_v] float32 or
    bfloat16; o_pre like h (float32 or bfloat16) or None; gamma, beta [H,d_v]
    float32 or None.  Returns y with h's dtype (``out`` may be h: in place)."""
    lib = load_library()
    h = _dev_tensor("h", h, (torch.float32, torch.bfloat16))
    if h.dim() != 4:
        raise ValueError("h must be [B,H,T,d_v]")
    B, H, T, dv = h.shape
    dev = h.device
    o_pre = _dev_tensor("o_pre", o_pre, (torch.float32, torch.bfloat16), (B, H, T, dv), dev)
    gamma = _dev_tensor("gamma", gamma, torch.float32, (H, dv), dev)
    beta = _dev_tensor("beta", beta, torch.float32, (H, dv), dev)
    y = (torch.empty_like(h) if out is None
         else _dev_tensor("out", out, h.dtype, (B, H, T, dv), dev))
    odt = _DT[o_pre.dtype] if o_pre is not None else MLSTM_F32
    _check(lib.mlstm_groupnorm_ogate(B, H, T, dv, _DT[h.dtype], odt, _ptr(h), _ptr(o_pre),
                                     _ptr(gamma), _ptr(beta), float(eps), _ptr(y),
                                     _stream_handle(stream)))
    return y


@_allocates_on_stream
def mlstm_causal_conv1d(x, w, bias=None, state=None, *, return_state: bool = True,
                        out: Optional[torch.Tensor] = None, stream=None):
    """Causal depthwise convolution over the token axis (see
    mlstm_causal_conv1d in include/mlstm.h).  x [B,T,C] float32 or bfloat16;
    w [C,K] float32; bias [C] float32 or None; state [B,K-1,C] float32 (the
    K-1 inputs before x[:,0]) or None.  Returns (y, new state) or (y, None)."""
    lib = load_library()
    x = _dev_tensor("x", x, (torch.float32, torch.bfloat16))
    if x.dim() != 3:
        raise ValueError("x must be [B,T,C]")
    B, T, C = x.shape
    dev = x.device
    w = _dev_tensor("w", w, torch.float32, None, dev)
    if w.dim() != 2 or w.shape[0] != C:
        raise ValueError(f"w must be [C={C},K]")
    K = w.shape[1]
    bias = _dev_tensor("bias", bias, torch.float32, (C,), dev)
    state = _dev_tensor("state", state, torch.float32, (B, K - 1, C), dev)
    y = (torch.empty_like(x) if out is None
         else _dev_tensor("out", out, x.dtype, (B, T, C), dev))
    st_out = torch.empty((B, K - 1, C), dtype=torch.float32, device=dev) if return_state else None
    _check(lib.mlstm_causal_conv1d(B, T, C, K, _DT[x.dtype], _ptr(x), _ptr(w), _ptr(bias),
                                   _ptr(state), _ptr(y), _ptr(st_out), _stream_handle(stream)))
    return y, st_out


class SlstmProblem(ctypes.Structure):
    """mlstm_slstm_problem_t."""
    _fields_ = [("B", ctypes.c_int64), ("NH", ctypes.c_int64), ("T", ctypes.c_int64),
                ("DH", ctypes.c_int64), ("x_dtype", ctypes.c_int32), ("fgate", ctypes.c_int32)]


@_allocates_on_stream
def mlstm_slstm_fwd(wx, R, c0=None, n0=None, m0=None, h0=None, *, fgate="sigmoid",
                    return_state: bool = True, out: Optional[torch.Tensor] = None, stream=None):
    """sLSTM forward cell (see mlstm_slstm_fwd in include/mlstm.h).

    wx [B,NH,T,4,DH] float32 or bfloat16 (gate order i, f, z, o); R
    [NH,4,DH,DH] float32; c0, n0, m0, h0 [B,NH,DH] float32 (all or none).
    Returns (h [B,NH,T,DH] in wx's dtype, (c1, n1, m1, h1)) or (h, None)."""
    lib = load_library()
    wx = _dev_tensor("wx", wx, (torch.float32, torch.bfloat16))
    if wx.dim() != 5 or wx.shape[3] != 4:
        raise ValueError("wx must be [B,NH,T,4,DH]")
    B, NH, T, _, DH = wx.shape
    dev = wx.device
    R = _dev_tensor("R", R, torch.float32, (NH, 4, DH, DH), dev)
    st = [_dev_tensor(nm, x, torch.float32, (B, NH, DH), dev)
          for nm, x in (("c0", c0), ("n0", n0), ("m0", m0), ("h0", h0))]
    h = (torch.empty((B, NH, T, DH), dtype=wx.dtype, device=dev) if out is None
         else _dev_tensor("out", out, wx.dtype, (B, NH, T, DH), dev))
    fin = ([torch.empty((B, NH, DH), dtype=torch.float32, device=dev) for _ in range(4)]
           if return_state else [None] * 4)
    p = SlstmProblem(B, NH, T, DH, _DT[wx.dtype], _fgate(fgate))
    _check(lib.mlstm_slstm_fwd(ctypes.byref(p), _ptr(wx), _ptr(R), *(_ptr(x) for x in st),
                               _ptr(h), *(_ptr(x) for x in fin), _stream_handle(stream)))
    return h, (tuple(fin) if return_state else None)
