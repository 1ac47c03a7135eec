"""fp64 CPU oracle for the mLSTM matrix-memory cell forward pass.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The HIP library
never links, loads or calls it, and it shares no code with the HIP library.

The arithmetic lives in ``mlstm_oracle.c`` (the plain sequential stabilized
recurrence of the xLSTM post, section 3 "Associative Matrix Cell State", with
the running maximum of section 2 "The Normalizer State and Numerical
Stabilization").  This module only builds that file with gcc, loads it with
ctypes and converts numpy arrays to contiguous float64 (an exact conversion
for both float32 and bfloat16 inputs).

Parity status: pinned.  The test suite checks the recurrence against the
unrolled-sum form evaluated in 50-digit arithmetic (``unrolled_mp``), against
a numpy fp64 evaluation of the quadratic parallel form, against causal linear
attention, against the closed form of the stabilizer, and against the
split/resume and stabilizer-shift invariants.

The gradient of the forward pass (``backward``) lives in
``mlstm_oracle_bwd.c``: reverse mode through the recurrence in true units.
Parity status: pinned, against central finite differences of the forward
recurrence, the closed form of one token, the closed form of causal linear
attention, and planted mistakes (``tests/test_oracle_bwd.py``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mlstm_oracle.c")
_SRC_BWD = os.path.join(_HERE, "mlstm_oracle_bwd.c")
_LIB = os.path.join(_HERE, "liboracle.so")

FGATE_SIGMOID = 0
FGATE_EXP = 1

_lib = None


def build() -> str:
    """Compile ``mlstm_oracle.c`` into ``liboracle.so`` next to it.

    No -ffast-math (it would allow reassociation) and no -march=native (the
    library travels to other hosts).
    """
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC, _SRC_BWD, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def build_variant(src_text: str, out_path: str, bwd_text: Optional[str] = None) -> str:
    """Compile an edited copy of the oracle source (used by the test that
    plants mistakes in the oracle to show that its pins catch them).
    ``bwd_text`` replaces the gradient source the same way (default: as is)."""
    src = out_path + ".c"
    with open(src, "w") as fh:
        fh.write(src_text)
    src_b = out_path + "_bwd.c"
    with open(src_b, "w") as fh:
        fh.write(bwd_source_text() if bwd_text is None else bwd_text)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                    "-o", out_path, src, src_b, "-lm"], check=True)
    return out_path


def source_text() -> str:
    with open(_SRC) as fh:
        return fh.read()


def bwd_source_text() -> str:
    with open(_SRC_BWD) as fh:
        return fh.read()


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if (not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)
            or os.path.getmtime(_LIB) < os.path.getmtime(_SRC_BWD)):
        build()
    _lib = load_library(_LIB)
    return _lib


def load_library(path: str):
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.oracle_recurrent.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int,
                                     P, P, P, P, P, P, P, P, P, P, P, P, P,
                                     ctypes.c_int]
    lib.oracle_recurrent.restype = None
    lib.oracle_step.argtypes = [i64, i64, i64, i64, ctypes.c_int,
                                P, P, P, P, P, P, P, P, P, P, ctypes.c_int]
    lib.oracle_step.restype = None
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_backward.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int] + [P] * 27 + [ctypes.c_int]
    lib.oracle_backward.restype = None
    return lib


def _f64(x) -> Optional[np.ndarray]:
    if x is None:
        return None
    if hasattr(x, "detach"):  # a torch tensor: widen on the torch side first
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def fgate_code(fgate) -> int:
    if fgate in (FGATE_SIGMOID, "sigmoid"):
        return FGATE_SIGMOID
    if fgate in (FGATE_EXP, "exp"):
        return FGATE_EXP
    raise ValueError(f"unknown forget gate {fgate!r}")


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def recurrent(q, k, v, i_pre, f_pre, o_pre=None, C0=None, n0=None, m0=None,
              fgate="sigmoid", nthreads: int = 0, lib=None):
    """Run the sequential recurrence over a whole sequence.

    Shapes: q, k [B,H,T,dqk]; v [B,H,T,dv]; i_pre, f_pre [B,H,T];
    o_pre [B,H,T,dv] or None; C0 [B,H,dqk,dv], n0 [B,H,dqk], m0 [B,H] or all
    None (zero state).  Returns (h [B,H,T,dv], C1, n1, m1) as float64 arrays.
    ``lib`` selects another build of the same source (default: liboracle.so).
    """
    lib = lib or _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    i_pre, f_pre, o_pre = _f64(i_pre), _f64(f_pre), _f64(o_pre)
    C0, n0, m0 = _f64(C0), _f64(n0), _f64(m0)
    if (C0 is None) != (n0 is None) or (C0 is None) != (m0 is None):
        raise ValueError("initial state must be given whole or not at all")
    B, H, T, dqk = q.shape
    dv = v.shape[-1]
    assert k.shape == (B, H, T, dqk) and v.shape == (B, H, T, dv)
    assert i_pre.shape == (B, H, T) and f_pre.shape == (B, H, T)
    if o_pre is not None:
        assert o_pre.shape == (B, H, T, dv)
    if C0 is not None:
        assert C0.shape == (B, H, dqk, dv) and n0.shape == (B, H, dqk)
        assert m0.shape == (B, H)
    h = np.empty((B, H, T, dv))
    C1 = np.empty((B, H, dqk, dv))
    n1 = np.empty((B, H, dqk))
    m1 = np.empty((B, H))
    lib.oracle_recurrent(B, H, T, dqk, dv, fgate_code(fgate), _ptr(q), _ptr(k),
                         _ptr(v), _ptr(i_pre), _ptr(f_pre), _ptr(o_pre),
                         _ptr(C0), _ptr(n0), _ptr(m0), _ptr(h), _ptr(C1),
                         _ptr(n1), _ptr(m1), int(nthreads))
    return h, C1, n1, m1


def step(q, k, v, i_pre, f_pre, o_pre, C, n, m, fgate="sigmoid",
         nthreads: int = 0, lib=None):
    """One token for every head.  q, k [B,H,dqk]; v [B,H,dv]; i_pre, f_pre
    [B,H]; o_pre [B,H,dv] or None; state C [B,H,dqk,dv], n [B,H,dqk], m [B,H].

    Returns (h, C', n', m') as new float64 arrays; the inputs are not changed.
    """
    lib = lib or _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    i_pre, f_pre, o_pre = _f64(i_pre), _f64(f_pre), _f64(o_pre)
    C, n, m = _f64(C).copy(), _f64(n).copy(), _f64(m).copy()
    B, H, dqk = q.shape
    dv = v.shape[-1]
    assert C.shape == (B, H, dqk, dv) and n.shape == (B, H, dqk)
    assert m.shape == (B, H) and i_pre.shape == (B, H)
    h = np.empty((B, H, dv))
    lib.oracle_step(B, H, dqk, dv, fgate_code(fgate), _ptr(q), _ptr(k), _ptr(v),
                    _ptr(i_pre), _ptr(f_pre), _ptr(o_pre), _ptr(C), _ptr(n),
                    _ptr(m), _ptr(h), int(nthreads))
    return h, C, n, m


def backward(q, k, v, i_pre, f_pre, o_pre, C0, n0, m0, dh, dC1=None, dn1=None,
             fgate="sigmoid", nthreads: int = 0, lib=None, h=None):
    """Gradient of L = sum dh . h + e^{-m_T} (<dC1, C_T> + <dn1, n_T>) (see
    ``mlstm_oracle_bwd.c``) with respect to every input of the forward pass.

    Shapes as in ``recurrent``; dh like v; dC1 [B,H,dqk,dv], dn1 [B,H,dqk] or
    both None.  ``h`` (like v, optional) is the forward output as a caller
    hands it to a backward pass; the gradient's two terms that depend on h
    itself (dh . h in the denominator term, and do~) then use it instead of
    the oracle's own fp64 h.  Returns a dict of float64 arrays: dq, dk, dv,
    di, df, do (None without o~), dC0, dn0, dm0 (the initial-state gradients
    in its stored scale; computed for the zero state too), and cond_dq,
    cond_dk, cond_di, cond_df, cond_dm0: the conditioning scale of dq, dk,
    di, df, dm0 (the sum of the absolute values of their memory and
    normalizer paths, which partly cancel on the active branch of the
    denominator).
    """
    lib = lib or _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    i_pre, f_pre, o_pre = _f64(i_pre), _f64(f_pre), _f64(o_pre)
    C0, n0, m0 = _f64(C0), _f64(n0), _f64(m0)
    dh, dC1, dn1, h = _f64(dh), _f64(dC1), _f64(dn1), _f64(h)
    if (C0 is None) != (n0 is None) or (C0 is None) != (m0 is None):
        raise ValueError("initial state must be given whole or not at all")
    if (dC1 is None) != (dn1 is None):
        raise ValueError("final-state gradient must be given whole or not at all")
    B, H, T, dqk = q.shape
    dv = v.shape[-1]
    assert dh.shape == (B, H, T, dv)
    if h is not None:
        assert h.shape == (B, H, T, dv)
    out = dict(dq=np.empty((B, H, T, dqk)), dk=np.empty((B, H, T, dqk)),
               dv=np.empty((B, H, T, dv)), di=np.empty((B, H, T)), df=np.empty((B, H, T)),
               do=None if o_pre is None else np.empty((B, H, T, dv)),
               dC0=np.empty((B, H, dqk, dv)), dn0=np.empty((B, H, dqk)), dm0=np.empty((B, H)),
               cond_dq=np.empty((B, H, T, dqk)), cond_dk=np.empty((B, H, T, dqk)),
               cond_di=np.empty((B, H, T)), cond_df=np.empty((B, H, T)),
               cond_dm0=np.empty((B, H)))
    lib.oracle_backward(B, H, T, dqk, dv, fgate_code(fgate), _ptr(q), _ptr(k), _ptr(v),
                        _ptr(i_pre), _ptr(f_pre), _ptr(o_pre), _ptr(C0), _ptr(n0), _ptr(m0),
                        _ptr(dh), _ptr(h), _ptr(dC1), _ptr(dn1), _ptr(out["dq"]),
                        _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["di"]), _ptr(out["df"]),
                        _ptr(out["do"]), _ptr(out["dC0"]), _ptr(out["dn0"]), _ptr(out["dm0"]),
                        _ptr(out["cond_dq"]), _ptr(out["cond_dk"]), _ptr(out["cond_di"]),
                        _ptr(out["cond_df"]), _ptr(out["cond_dm0"]),
                        int(nthreads))
    return out
