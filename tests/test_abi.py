"""The C ABI on the host (no GPU needed): the library loads, exports every
function include/mlstm.h declares, and rejects invalid calls with the
documented status before anything is enqueued.  Every call here fails its
checks, so no kernel is launched."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import mlstm_matrix_memory_chunkwise_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mlstm.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(M.library_path()):
        pytest.fail("libmlstm.so is not built (run __graft_entry__.build())")
    return M.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mlstm_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("mlstm_fwd_chunkwise", "mlstm_fwd_parallel", "mlstm_step",
              "mlstm_fwd_chunkwise_workspace_bytes", "mlstm_fwd_parallel_workspace_bytes",
              "mlstm_status_string", "mlstm_last_error_detail", "mlstm_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} not exported"


def test_library_exports_nothing_else():
    """The only C-linkage functions of the library are the declared entry
    points (C++ helpers carry mangled names; the HIP runtime adds its
    per-module ids)."""
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", M.library_path()], capture_output=True,
                         text=True, check=True).stdout
    names = {line.split()[-1] for line in out.splitlines() if line.strip()}
    plain = {n for n in names if not n.startswith("_Z") and not n.startswith("__hip_cuid")}
    assert plain == set(declared_functions()), plain ^ set(declared_functions())


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "mlstm.h"\nint main(void){ mlstm_problem_t p; (void)p; '
                   'return (int)sizeof(mlstm_problem_t) == 56 ? 0 : 1; }\n')
    import subprocess
    exe = tmp_path / "t"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe)], check=True)
    assert subprocess.run([str(exe)]).returncode == 0
    assert ctypes.sizeof(M.Problem) == 56


def test_status_strings(lib):
    assert lib.mlstm_status_string(0) == b"ok"
    assert lib.mlstm_status_string(1) == b"invalid argument"
    assert lib.mlstm_status_string(2) == b"unsupported problem"
    assert lib.mlstm_status_string(3) == b"device error"
    assert M.mlstm_version().startswith("mlstm-gfx950")


def P(B=1, H=1, T=64, dqk=16, dv=16, qkv=0, o=0, fg=0, res=0):
    return M.Problem(B, H, T, dqk, dv, qkv, o, fg, res)


FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails its checks


def ptrs(n, base=FAKE, stride=1 << 30):
    return [ctypes.c_void_p(base + i * stride) for i in range(n)]


def chunk_call(lib, p, chunk=16, **over):
    names = ["q", "k", "v", "i", "f", "o", "C0", "n0", "m0", "h", "C1", "n1", "m1"]
    vals = dict(zip(names, ptrs(len(names))))
    vals["o"] = None
    vals["C0"] = vals["n0"] = vals["m0"] = None
    vals["C1"] = vals["n1"] = vals["m1"] = None
    vals.update(over)
    r = lib.mlstm_fwd_chunkwise(ctypes.byref(p), chunk, *(vals[n] for n in names), None, 0, None)
    return r, lib.mlstm_last_error_detail().decode()


def test_chunkwise_rejects_missing_pointers(lib):
    for name in ("q", "k", "v", "i", "f", "h"):
        r, det = chunk_call(lib, P(), **{name: None, "q": None if name == "q" else ctypes.c_void_p(FAKE)})
        assert r == M.MLSTM_ERR_INVALID_ARG, (name, det)


def test_chunkwise_rejects_partial_state(lib):
    p = P()
    r, det = chunk_call(lib, p, C0=ctypes.c_void_p(FAKE + 20 * (1 << 30)))
    assert r == M.MLSTM_ERR_INVALID_ARG and "initial state" in det
    r, det = chunk_call(lib, p, C1=ctypes.c_void_p(FAKE + 20 * (1 << 30)),
                        n1=ctypes.c_void_p(FAKE + 21 * (1 << 30)))
    assert r == M.MLSTM_ERR_INVALID_ARG and "final state" in det


@pytest.mark.parametrize("field,value", [("B", -1), ("H", -1), ("T", -1), ("d_qk", 0), ("d_v", 0)])
def test_chunkwise_rejects_bad_sizes(lib, field, value):
    p = P()
    setattr(p, field, value)
    r, _ = chunk_call(lib, p)
    assert r == M.MLSTM_ERR_INVALID_ARG


@pytest.mark.parametrize("field", ["B", "H", "T"])
def test_empty_sequences_are_no_ops(lib, field):
    """B*H = 0 or T = 0: nothing to compute, every per-token pointer may be
    NULL, and without state pointers nothing is enqueued (so this runs without
    a GPU)."""
    p = P()
    setattr(p, field, 0)
    none = [None] * 13
    assert lib.mlstm_fwd_chunkwise(ctypes.byref(p), 16, *none, None, 0, None) == 0
    assert lib.mlstm_fwd_parallel(ctypes.byref(p), *none, None, 0, None) == 0
    n = ctypes.c_size_t(7)
    assert lib.mlstm_fwd_chunkwise_workspace_bytes(ctypes.byref(p), 64, ctypes.byref(n)) == 0
    assert n.value == 0
    assert lib.mlstm_bwd_chunkwise_workspace_bytes(ctypes.byref(p), 16, ctypes.byref(n)) == 0
    assert n.value == 0
    if field != "T":   # no heads: the backward and the step do nothing either
        assert lib.mlstm_bwd_chunkwise(ctypes.byref(p), 16, *([None] * 22), None, 0, None) == 0
        assert lib.mlstm_step(ctypes.byref(p), *([None] * 14), None) == 0
    # partial state is still an error
    r = lib.mlstm_fwd_chunkwise(ctypes.byref(p), 16, *([None] * 6), ctypes.c_void_p(FAKE),
                                *([None] * 6), None, 0, None)
    assert r == M.MLSTM_ERR_INVALID_ARG or field != "T"



def test_chunkwise_rejects_bad_enums(lib):
    for kw in (dict(qkv=7), dict(o=3), dict(fg=2), dict(res=1)):
        r, _ = chunk_call(lib, P(**kw))
        assert r == M.MLSTM_ERR_INVALID_ARG, kw


def test_chunkwise_unsupported(lib):
    assert chunk_call(lib, P(dqk=24))[0] == M.MLSTM_ERR_UNSUPPORTED
    assert chunk_call(lib, P(dv=528))[0] == M.MLSTM_ERR_UNSUPPORTED
    assert chunk_call(lib, P(T=64), chunk=48)[0] == M.MLSTM_ERR_UNSUPPORTED


def test_chunkwise_ragged_T_workspace(lib):
    """T = 72 at chunk 64 on the bf16 matrix-core path: the last 8 tokens
    continue from the state of the first 64, which the workspace holds, so a
    call without one is refused before anything is launched."""
    n = ctypes.c_size_t(0)
    p = P(B=2, H=3, T=72, dqk=64, dv=64, qkv=1)
    assert lib.mlstm_fwd_chunkwise_workspace_bytes(ctypes.byref(p), 64, ctypes.byref(n)) == 0
    assert n.value == 4 * 6 * (64 * 64 + 64 + 1)
    r, det = chunk_call(lib, p, chunk=64)
    assert r == M.MLSTM_ERR_INVALID_ARG and "workspace" in det
    # a workspace placed over h is refused too
    names = ["q", "k", "v", "i", "f", "o", "C0", "n0", "m0", "h", "C1", "n1", "m1"]
    vals = dict(zip(names, ptrs(len(names))))
    vals.update(o=None, C0=None, n0=None, m0=None, C1=None, n1=None, m1=None)
    r = lib.mlstm_fwd_chunkwise(ctypes.byref(p), 64, *(vals[k] for k in names),
                                vals["h"], n.value, None)
    assert r == M.MLSTM_ERR_INVALID_ARG
    assert "workspace overlaps h" in lib.mlstm_last_error_detail().decode()
    # no carried state is needed for a multiple of the chunk, for T below one
    # chunk, or on the float32 path (one kernel takes the short last chunk)
    for q, chunk in ((P(T=128, dqk=64, dv=64, qkv=1), 64), (P(T=40, dqk=64, dv=64, qkv=1), 64),
                     (P(T=72), 16)):
        assert lib.mlstm_fwd_chunkwise_workspace_bytes(ctypes.byref(q), chunk, ctypes.byref(n)) == 0
        assert n.value == 0


def test_chunkwise_rejects_misalignment(lib):
    r, det = chunk_call(lib, P(), k=ctypes.c_void_p(FAKE + (1 << 30) + 8))
    assert r == M.MLSTM_ERR_INVALID_ARG and "aligned" in det


def test_chunkwise_rejects_overlaps(lib):
    # h placed inside q
    r, det = chunk_call(lib, P(), h=ctypes.c_void_p(FAKE + 64))
    assert r == M.MLSTM_ERR_INVALID_ARG and "overlaps" in det
    # final state written over the initial state
    st = FAKE + 40 * (1 << 30)
    r, det = chunk_call(lib, P(), C0=ctypes.c_void_p(st), n0=ctypes.c_void_p(st + (1 << 20)),
                        m0=ctypes.c_void_p(st + (2 << 20)), C1=ctypes.c_void_p(st),
                        n1=ctypes.c_void_p(st + (3 << 20)), m1=ctypes.c_void_p(st + (4 << 20)))
    assert r == M.MLSTM_ERR_INVALID_ARG and "overlaps" in det


def test_workspace_queries(lib):
    n = ctypes.c_size_t(123)
    assert lib.mlstm_fwd_chunkwise_workspace_bytes(ctypes.byref(P()), 16, ctypes.byref(n)) == 0
    assert n.value == 0
    assert lib.mlstm_fwd_chunkwise_workspace_bytes(ctypes.byref(P()), 17, ctypes.byref(n)) == \
        M.MLSTM_ERR_UNSUPPORTED
    assert lib.mlstm_fwd_parallel_workspace_bytes(ctypes.byref(P(B=2, H=3, T=100)),
                                                  ctypes.byref(n)) == 0
    assert n.value == 8 * 3 * 2 * 3 * 100
    assert lib.mlstm_fwd_parallel_workspace_bytes(None, ctypes.byref(n)) == M.MLSTM_ERR_INVALID_ARG


def test_parallel_requires_workspace(lib):
    v = ptrs(13)
    r = lib.mlstm_fwd_parallel(ctypes.byref(P()), v[0], v[1], v[2], v[3], v[4], None, None, None,
                               None, v[9], None, None, None, None, 0, None)
    assert r == M.MLSTM_ERR_INVALID_ARG
    assert "workspace" in lib.mlstm_last_error_detail().decode()


def step_call(lib, p, **over):
    names = ["q", "k", "v", "i", "f", "o", "Ci", "ni", "mi", "Co", "no", "mo", "h"]
    vals = dict(zip(names, ptrs(len(names))))
    vals["o"] = None
    vals.update(over)
    r = lib.mlstm_step(ctypes.byref(p), *(vals[n] for n in names), None)
    return r, lib.mlstm_last_error_detail().decode()


def test_step_rejects_missing_state(lib):
    for name in ("Ci", "ni", "mi", "Co", "no", "mo", "h", "q"):
        r, _ = step_call(lib, P(), **{name: None})
        assert r == M.MLSTM_ERR_INVALID_ARG, name


def test_step_in_place_rules(lib):
    base = ptrs(13)
    # exact aliasing of each state output with its input is allowed by the
    # checks; the call then reaches the launch, which we must not do here, so
    # only partial overlap and cross aliasing are exercised
    r, det = step_call(lib, P(), Co=ctypes.c_void_p(base[6].value + 16))
    assert r == M.MLSTM_ERR_INVALID_ARG and "overlaps" in det
    r, det = step_call(lib, P(), no=base[6])          # n_out inside C_in
    assert r == M.MLSTM_ERR_INVALID_ARG and "overlaps" in det
    r, det = step_call(lib, P(), h=base[0])           # h over q
    assert r == M.MLSTM_ERR_INVALID_ARG and "overlaps" in det


def test_python_binding_refuses_host_tensors():
    import torch
    q = torch.zeros(1, 1, 16, 16)
    with pytest.raises(ValueError):
        M.mlstm_fwd_chunkwise(q, q, q, torch.zeros(1, 1, 16), torch.zeros(1, 1, 16), chunk=16)


BWD_NAMES = ["q", "k", "v", "i", "f", "o", "C0", "n0", "m0", "h", "dh", "dC1", "dn1",
             "dq", "dk", "dv", "di", "df", "do", "dC0", "dn0", "dm0"]


def bwd_call(lib, p, chunk=16, ws_bytes=1 << 40, **over):
    vals = dict(zip(BWD_NAMES, ptrs(len(BWD_NAMES))))
    for n in ("o", "C0", "n0", "m0", "dC1", "dn1", "do", "dC0", "dn0", "dm0"):
        vals[n] = None
    vals.update(over)
    ws = over.get("ws", ctypes.c_void_p(FAKE + 60 * (1 << 30)))
    r = lib.mlstm_bwd_chunkwise(ctypes.byref(p), chunk, *(vals[n] for n in BWD_NAMES), ws,
                                ws_bytes, None)
    return r, lib.mlstm_last_error_detail().decode()


def test_bwd_rejects_missing_pointers(lib):
    for name in ("q", "k", "v", "i", "f", "h", "dh", "dq", "dk", "dv", "di", "df"):
        r, det = bwd_call(lib, P(), **{name: None})
        assert r == M.MLSTM_ERR_INVALID_ARG, (name, det)


def test_bwd_pairing_rules(lib):
    r, det = bwd_call(lib, P(), o=ctypes.c_void_p(FAKE + 30 * (1 << 30)))
    assert r == M.MLSTM_ERR_INVALID_ARG and "d_o" in det
    r, det = bwd_call(lib, P(), dC1=ctypes.c_void_p(FAKE + 30 * (1 << 30)))
    assert r == M.MLSTM_ERR_INVALID_ARG and "final-state gradient" in det
    r, det = bwd_call(lib, P(), C0=ctypes.c_void_p(FAKE + 30 * (1 << 30)))
    assert r == M.MLSTM_ERR_INVALID_ARG and "initial state" in det


def test_bwd_ragged_T_workspace(lib):
    """T not a multiple of the chunk: the pass runs on 14 per-token arrays
    padded to the next multiple Tp at the front of the workspace, followed by
    the workspace of the padded problem.  Without room for them the call is
    refused before anything is launched."""
    n, n_pad = ctypes.c_size_t(0), ctypes.c_size_t(0)
    for p, pp, chunk in ((P(T=96, dqk=64, dv=64, qkv=1), P(T=128, dqk=64, dv=64, qkv=1), 64),
                         (P(T=40), P(T=48), 16)):
        assert lib.mlstm_bwd_chunkwise_workspace_bytes(ctypes.byref(p), chunk, ctypes.byref(n)) == 0
        assert lib.mlstm_bwd_chunkwise_workspace_bytes(ctypes.byref(pp), chunk,
                                                       ctypes.byref(n_pad)) == 0
        sq, so = (2 if p.qkv_dtype else 4), 4
        rows = [p.d_qk * sq] * 2 + [p.d_v * sq, 4, 4, p.d_v * so, p.d_v * sq, p.d_v * sq,
                                    p.d_qk * 4, p.d_qk * 4, p.d_v * 4, 4, 4, p.d_v * 4]
        pad = sum((pp.T * r + 255) // 256 * 256 for r in rows)
        assert n.value == pad + n_pad.value
        r, det = bwd_call(lib, p, chunk=chunk, ws_bytes=n.value - 1)
        assert r == M.MLSTM_ERR_INVALID_ARG and "workspace" in det


def test_bwd_unsupported(lib):
    # chunk 64 is the MFMA path: bf16 q/k/v, d_v % 64 == 0, d_qk in {64, 128, 256}
    assert bwd_call(lib, P(), chunk=64)[0] == M.MLSTM_ERR_UNSUPPORTED
    assert bwd_call(lib, P(dqk=64, dv=64), chunk=64)[0] == M.MLSTM_ERR_UNSUPPORTED
    assert bwd_call(lib, P(dqk=96, dv=64, qkv=1), chunk=64)[0] == M.MLSTM_ERR_UNSUPPORTED
    assert bwd_call(lib, P(dqk=64, dv=32, qkv=1), chunk=64)[0] == M.MLSTM_ERR_UNSUPPORTED
    assert bwd_call(lib, P(), chunk=128)[0] == M.MLSTM_ERR_UNSUPPORTED
    assert bwd_call(lib, P(dqk=512, dv=32))[0] == M.MLSTM_ERR_UNSUPPORTED
    assert bwd_call(lib, P(dqk=272, dv=48))[0] == M.MLSTM_ERR_UNSUPPORTED


def test_bwd_alignment(lib):
    """h and dh are read in 16-byte pieces at every chunk; chunk 64 moves the
    other [.., d_v] arrays that way too (4-byte aligned dv is accepted by
    chunk 32 only)."""
    p = P(dqk=64, dv=64, qkv=1)
    odd_dh = ctypes.c_void_p(FAKE + 10 * (1 << 30) + 4)
    for chunk in (32, 64):
        r, det = bwd_call(lib, p, chunk=chunk, dh=odd_dh)
        assert r == M.MLSTM_ERR_INVALID_ARG and "dh" in det and "aligned" in det
    odd_dq = ctypes.c_void_p(FAKE + 13 * (1 << 30) + 4)
    r, det = bwd_call(lib, p, chunk=32, dq=odd_dq)
    assert r == M.MLSTM_ERR_INVALID_ARG and "dq" in det and "aligned" in det
    odd_dv = ctypes.c_void_p(FAKE + 15 * (1 << 30) + 4)
    r, det = bwd_call(lib, p, chunk=64, dv=odd_dv)
    assert r == M.MLSTM_ERR_INVALID_ARG and "dv" in det and "aligned" in det
    r, det = bwd_call(lib, p, chunk=32, dv=odd_dv, ws_bytes=0)
    assert r == M.MLSTM_ERR_INVALID_ARG and "workspace" in det


def test_bwd_workspace(lib):
    n = ctypes.c_size_t(0)
    p = P(B=2, H=3, T=64, dqk=16, dv=16)
    assert lib.mlstm_bwd_chunkwise_workspace_bytes(ctypes.byref(p), 16, ctypes.byref(n)) == 0
    # the stored boundary states and the per-column-block partials dominate
    assert n.value >= 2 * 3 * (64 // 16 + 1) * 16 * 16 * 4 + 2 * 1 * 2 * 3 * 64 * 16 * 4
    r, det = bwd_call(lib, p, ws_bytes=n.value - 1)
    assert r == M.MLSTM_ERR_INVALID_ARG and "workspace" in det
    r, det = bwd_call(lib, p, ws=ctypes.c_void_p(FAKE + 64))   # inside q
    assert r == M.MLSTM_ERR_INVALID_ARG and "overlaps" in det


# ---- block operations (no kernel runs: every call below fails its checks)

def gn_call(lib, B=1, H=2, T=4, dv=64, hdt=1, odt=0, eps=1e-5, **over):
    v = dict(h=ctypes.c_void_p(FAKE), o=None, g=None, b=None, y=ctypes.c_void_p(FAKE + (1 << 30)))
    v.update(over)
    r = lib.mlstm_groupnorm_ogate(B, H, T, dv, hdt, odt, v["h"], v["o"], v["g"], v["b"],
                                  ctypes.c_float(eps), v["y"], None)
    return r, lib.mlstm_last_error_detail().decode()


def test_groupnorm_rejections(lib):
    assert gn_call(lib, h=None)[0] == M.MLSTM_ERR_INVALID_ARG
    assert gn_call(lib, y=None)[0] == M.MLSTM_ERR_INVALID_ARG
    assert gn_call(lib, T=-1)[0] == M.MLSTM_ERR_INVALID_ARG
    assert gn_call(lib, T=0, h=None, y=None)[0] == 0   # no rows: nothing to do
    r, det = gn_call(lib, B=2, H=1 << 16, T=(1 << 15) + 1)
    assert r == M.MLSTM_ERR_UNSUPPORTED and "2^32" in det
    assert gn_call(lib, hdt=7)[0] == M.MLSTM_ERR_INVALID_ARG
    assert gn_call(lib, eps=-1.0)[0] == M.MLSTM_ERR_INVALID_ARG
    assert gn_call(lib, eps=float("nan"))[0] == M.MLSTM_ERR_INVALID_ARG
    assert gn_call(lib, dv=6)[0] == M.MLSTM_ERR_UNSUPPORTED
    assert gn_call(lib, dv=2048)[0] == M.MLSTM_ERR_UNSUPPORTED
    r, det = gn_call(lib, o=ctypes.c_void_p(FAKE + (2 << 30) + 8))   # rows move in 16-byte pieces
    assert r == M.MLSTM_ERR_INVALID_ARG and "o_pre" in det
    r, det = gn_call(lib, y=ctypes.c_void_p(FAKE + 64))              # inside h, not h
    assert r == M.MLSTM_ERR_INVALID_ARG and "overlaps" in det
    r, det = gn_call(lib, g=ctypes.c_void_p(FAKE + (1 << 30) + 128))  # gamma inside y
    assert r == M.MLSTM_ERR_INVALID_ARG and "overlaps" in det


def conv_call(lib, B=1, T=16, C=64, K=4, dt=1, **over):
    names = ["x", "w", "bias", "sin", "y", "sout"]
    v = dict(zip(names, ptrs(len(names))))
    v["bias"] = v["sin"] = v["sout"] = None
    v.update(over)
    r = lib.mlstm_causal_conv1d(B, T, C, K, dt, *(v[n] for n in names), None)
    return r, lib.mlstm_last_error_detail().decode()


def test_conv_rejections(lib):
    for n in ("x", "w", "y"):
        assert conv_call(lib, **{n: None})[0] == M.MLSTM_ERR_INVALID_ARG, n
    assert conv_call(lib, K=0)[0] == M.MLSTM_ERR_INVALID_ARG
    assert conv_call(lib, T=-1)[0] == M.MLSTM_ERR_INVALID_ARG
    assert conv_call(lib, B=0, x=None, w=None, y=None)[0] == 0   # nothing to do
    assert conv_call(lib, T=0, x=None, y=None)[0] == 0           # no window to carry
    assert conv_call(lib, dt=3)[0] == M.MLSTM_ERR_INVALID_ARG
    assert conv_call(lib, K=9)[0] == M.MLSTM_ERR_UNSUPPORTED
    assert conv_call(lib, C=12)[0] == M.MLSTM_ERR_UNSUPPORTED            # bf16: C % 8
    assert conv_call(lib, C=12, dt=0, x=None)[0] == M.MLSTM_ERR_INVALID_ARG
    r, det = conv_call(lib, x=ctypes.c_void_p(FAKE + 8))
    assert r == M.MLSTM_ERR_INVALID_ARG and "aligned" in det
    r, det = conv_call(lib, sout=ctypes.c_void_p(FAKE + 16))             # inside x
    assert r == M.MLSTM_ERR_INVALID_ARG and "overlaps" in det
    r, det = conv_call(lib, sin=ctypes.c_void_p(FAKE + (4 << 30)),
                       sout=ctypes.c_void_p(FAKE + (4 << 30)))          # in place is refused
    assert r == M.MLSTM_ERR_INVALID_ARG and "overlaps" in det


# ---- sLSTM cell

def test_slstm_problem_layout(tmp_path):
    src = tmp_path / "s.c"
    src.write_text('#include "mlstm.h"\nint main(void){ return sizeof(mlstm_slstm_problem_t) == 40 ? 0 : 1; }\n')
    import subprocess
    exe = tmp_path / "s"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe)], check=True)
    assert subprocess.run([str(exe)]).returncode == 0
    assert ctypes.sizeof(M.SlstmProblem) == 40


def slstm_call(lib, B=2, NH=2, T=8, DH=32, dt=0, fg=0, **over):
    names = ["wx", "R", "c0", "n0", "m0", "h0", "h", "c1", "n1", "m1", "h1"]
    v = dict(zip(names, ptrs(len(names))))
    for n in ("c0", "n0", "m0", "h0", "c1", "n1", "m1", "h1"):
        v[n] = None
    v.update(over)
    p = M.SlstmProblem(B, NH, T, DH, dt, fg)
    r = lib.mlstm_slstm_fwd(ctypes.byref(p), *(v[n] for n in names), None)
    return r, lib.mlstm_last_error_detail().decode()


def test_slstm_rejections(lib):
    for n in ("wx", "R", "h"):
        assert slstm_call(lib, **{n: None})[0] == M.MLSTM_ERR_INVALID_ARG, n
    assert slstm_call(lib, T=-1)[0] == M.MLSTM_ERR_INVALID_ARG
    # no steps and no state: nothing to do (state pointers are None by default)
    assert slstm_call(lib, T=0, wx=None, R=None, h=None)[0] == 0
    assert slstm_call(lib, B=0, wx=None, R=None, h=None)[0] == 0
    assert slstm_call(lib, dt=5)[0] == M.MLSTM_ERR_INVALID_ARG
    assert slstm_call(lib, fg=9)[0] == M.MLSTM_ERR_INVALID_ARG
    assert slstm_call(lib, DH=48)[0] == M.MLSTM_ERR_UNSUPPORTED
    assert slstm_call(lib, DH=256)[0] == M.MLSTM_ERR_UNSUPPORTED
    r, det = slstm_call(lib, c0=ctypes.c_void_p(FAKE + (2 << 30)))
    assert r == M.MLSTM_ERR_INVALID_ARG and "initial state" in det
    r, det = slstm_call(lib, c1=ctypes.c_void_p(FAKE + (7 << 30)))
    assert r == M.MLSTM_ERR_INVALID_ARG and "final state" in det
    r, det = slstm_call(lib, R=ctypes.c_void_p(FAKE + (1 << 30) + 4))
    assert r == M.MLSTM_ERR_INVALID_ARG and "R" in det and "aligned" in det
    r, det = slstm_call(lib, h=ctypes.c_void_p(FAKE + 64))                # inside wx
    assert r == M.MLSTM_ERR_INVALID_ARG and "overlaps" in det


def test_noalloc_rejects_problems_beyond_its_scratch(lib):
    """mlstm_fwd_chunkwise_noalloc: a ragged bf16 problem whose carried state
    (B*H*(d_qk*d_v + d_qk + 1) floats) exceeds the fixed 64 MiB scratch is
    refused on the host with MLSTM_ERR_UNSUPPORTED, naming the size; one that
    fits gets past that check (and here, without a GPU, fails on the device
    lookup instead)."""
    names = ["q", "k", "v", "i", "f", "o", "C0", "n0", "m0", "h", "C1", "n1", "m1"]

    def call(p):
        vals = dict(zip(names, ptrs(len(names))))
        for n in ("o", "C0", "n0", "m0", "C1", "n1", "m1"):
            vals[n] = None
        r = lib.mlstm_fwd_chunkwise_noalloc(ctypes.byref(p), 64, *(vals[n] for n in names), None)
        return r, lib.mlstm_last_error_detail().decode()

    big = P(B=1, H=128, T=129, dqk=256, dv=512, qkv=1)
    need = M.mlstm_fwd_chunkwise_workspace_bytes(big, 64)
    assert need > 64 << 20
    r, det = call(big)
    assert r == M.MLSTM_ERR_UNSUPPORTED and str(need) in det and "noalloc" in det, det
    # a problem without a tail needs no scratch at all; nor does an empty one
    assert M.mlstm_fwd_chunkwise_workspace_bytes(P(B=1, H=128, T=128, dqk=256, dv=512, qkv=1),
                                                 64) == 0
    small = P(B=1, H=2, T=129, dqk=256, dv=512, qkv=1)
    r, det = call(small)
    if not torch_has_gpu():
        assert r == M.MLSTM_ERR_DEVICE, det


def torch_has_gpu():
    import torch
    return torch.cuda.is_available()


def test_sequence_split_plan():
    """A chunkwise call whose grid (B*H*d_v/64 workgroups) covers at most 128
    compute units and whose halves are at least 2048 tokens (whole chunks and
    multiples of 64) runs as two halves: the workspace holds the half-heads'
    states.  Larger grids, short or ragged sequences, and the float32 path do
    not split (no workspace when T is a multiple of the chunk)."""
    ws = lambda p, c: M.mlstm_fwd_chunkwise_workspace_bytes(p, c)  # noqa: E731
    BH, dqk, dv = 16, 256, 512
    state = BH * (dqk * dv + dqk + 1) * 4
    assert ws(P(B=1, H=16, T=65536, dqk=256, dv=512, qkv=1), 128) >= 5 * state
    assert ws(P(B=1, H=2, T=4096, dqk=256, dv=128, qkv=1), 64) > 0
    assert ws(P(B=8, H=8, T=8192, dqk=256, dv=256, qkv=1), 64) == 0     # 256 workgroups
    assert ws(P(B=1, H=2, T=2048, dqk=256, dv=128, qkv=1), 64) == 0     # halves too short
    assert ws(P(B=1, H=2, T=4096 + 64, dqk=256, dv=128, qkv=1), 64) == 0   # halves not multiples of 64
    assert ws(P(B=1, H=2, T=4096, dqk=256, dv=128, qkv=0), 64) == 0     # float32 path
