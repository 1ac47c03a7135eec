"""GPU parity of the chunkwise backward pass (mlstm_bwd_chunkwise) against the
fp64 gradient oracle (oracle.backward, pinned in test_oracle_bwd.py).

Both sides get the same inputs, the forward output h included: h is the
oracle's fp64 forward output rounded to the dtype of q/k/v, the value a
forward pass in that dtype hands over.  (The gradient is ill-conditioned in
h: in an exponential-gate recipe without o-gate, rounding the exact h to
bf16 alone moves di by 2e-2 and dq, dk by up to 1.7e-2.  Handing both sides
the same h removes that from the comparison.)

Every gradient is compared per (batch, head) slice.  dv, do, dC0 and dn0 use
the normwise relative error max|x - r| / max|r|.  dq, dk, di, df and dm0 are
each the sum of a memory path and a normalizer path, which partly cancel on
the active branch of the denominator; they use max|x - r| / max(cond), with
cond the oracle's sum of the two paths' absolute values (cond >= |r|, equal
where nothing cancels).  The plain normwise error and the elementwise
diagnostic are logged beside it.

dm0 = <dC0, C~0> + <dn0, n~0> is an inner product over every entry of the
state, so it amplifies the (normwise small) error of dC0 and dn0 by the
ratio of their largest to their typical entries: against the oracle it
measures that ratio more than the kernel.  It is checked in two parts: the
kernel's dm0 equals the inner product of its own dC0, dn0 with the initial
state (to float32 summation accuracy), and dC0, dn0 match the oracle like
every other gradient.  Its error against the oracle is logged.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from helpers import (TOL_BF16, TOL_F32, elem_rel_err, f64, gather_heads, has_gpu, log, sample_heads,
                     slice_rel_err, to_dev)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]


def _M():
    import mlstm_matrix_memory_chunkwise_amd as M
    return M


def make_inputs(seed, dtype, B, H, T, dqk, dv, *, o=True, state=True, dstate=True,
                i_dist=(-2.0, 3.0), f_dist=(4.0, 2.0)):
    g = torch.Generator().manual_seed(seed)
    n = lambda *s, mu=0.0, sd=1.0: torch.randn(*s, generator=g) * sd + mu  # noqa: E731
    inp = dict(
        q=n(B, H, T, dqk).to(dtype),
        k=(n(B, H, T, dqk) / dqk ** 0.5).to(dtype),
        v=n(B, H, T, dv).to(dtype),
        i_pre=n(B, H, T, mu=i_dist[0], sd=i_dist[1]),
        f_pre=n(B, H, T, mu=f_dist[0], sd=f_dist[1]),
        o_pre=n(B, H, T, dv) if o else None,
        C0=n(B, H, dqk, dv) if state else None,
        n0=n(B, H, dqk) if state else None,
        m0=n(B, H) if state else None,
    )
    grads_in = dict(dh=n(B, H, T, dv).to(dtype),
                    dC1=n(B, H, dqk, dv) if dstate else None,
                    dn1=n(B, H, dqk) if dstate else None)
    return inp, grads_in


def oracle_h(inp, fgate, o_dtype, heads=None):
    """The oracle's forward output of (the selected heads of) the inputs,
    rounded to the dtype of q/k/v."""
    sel = (lambda t: t) if heads is None else (lambda t: gather_heads(t, heads))
    x = {k: (None if v is None else sel(v)) for k, v in inp.items()}
    o = None if x["o_pre"] is None else x["o_pre"].to(o_dtype)
    h, *_ = oracle.recurrent(x["q"], x["k"], x["v"], x["i_pre"], x["f_pre"], o, x["C0"], x["n0"],
                             x["m0"], fgate=fgate)
    return torch.from_numpy(h).to(inp["q"].dtype)


def run_gpu(inp, gin, chunk, fgate, o_dtype, h):
    M = _M()
    d = to_dev(inp)
    gd = to_dev(gin)
    o = None if d["o_pre"] is None else d["o_pre"].to(o_dtype)
    g = M.mlstm_bwd_chunkwise(d["q"], d["k"], d["v"], d["i_pre"], d["f_pre"], o,
                              d["C0"], d["n0"], d["m0"], h.to("cuda"), gd["dh"], gd["dC1"],
                              gd["dn1"], chunk=chunk, fgate=fgate)
    torch.cuda.synchronize()
    return {k: (None if v is None else v.cpu()) for k, v in g.items()}


def run_oracle(inp, gin, fgate, o_dtype, h, heads=None):
    sel = (lambda t: t) if heads is None else (lambda t: gather_heads(t, heads))
    x = {k: (None if v is None else sel(v)) for k, v in {**inp, **gin}.items()}
    o = None if x["o_pre"] is None else x["o_pre"].to(o_dtype)
    return oracle.backward(x["q"], x["k"], x["v"], x["i_pre"], x["f_pre"], o, x["C0"], x["n0"],
                           x["m0"], x["dh"], x["dC1"], x["dn1"], fgate=fgate, h=h)


# gradients that are the sum of a memory and a normalizer path
PATHS = ("dq", "dk", "di", "df")
# dm0 against the inner product of the kernel's own dC0, dn0 with the state:
# float32 sums over d_qk*d_v terms
DM0_CONSISTENCY = 1e-4


def cond_rel_err(x, r, cond, lead):
    """max over slices of max|x - r| / max(cond)."""
    x, r, c = f64(x), f64(r), f64(cond)
    if np.isnan(x).any():
        return float("inf")
    n = int(np.prod(x.shape[:lead]))
    xs, rs, cs = x.reshape(n, -1), r.reshape(n, -1), c.reshape(n, -1)
    return float(np.max(np.max(np.abs(xs - rs), axis=1) / np.maximum(np.max(cs, axis=1), 1e-300)))


def dm0_consistency(g, C0, n0, heads=None):
    """max over heads of |dm0 - (<dC0, C~0> + <dn0, n~0>)| / sum of |terms|,
    the inner products taken in fp64 from the kernel's own dC0, dn0."""
    sel = (lambda t: t) if heads is None else (lambda t: gather_heads(t, heads))
    dC0, dn0, dm0 = f64(sel(g["dC0"])), f64(sel(g["dn0"])), f64(sel(g["dm0"]))
    C0, n0 = f64(sel(C0)), f64(sel(n0))
    ip = (dC0 * C0).sum((2, 3)) + (dn0 * n0).sum(2)
    mag = np.abs(dC0 * C0).sum((2, 3)) + np.abs(dn0 * n0).sum(2)
    if np.isnan(dm0).any():
        return float("inf")
    return float(np.max(np.abs(dm0 - ip) / np.maximum(mag, 1e-300)))


def compare(g, r, tol, label, state, heads=None, C0=None, n0=None):
    names = ["dq", "dk", "dv", "di", "df"] + (["do"] if r["do"] is not None else [])
    names += ["dC0", "dn0"]
    errs, plain, elem = {}, {}, {}
    for nme in names:
        x = g[nme] if heads is None else gather_heads(g[nme], heads)
        ref = r[nme]
        plain[nme] = slice_rel_err(x, ref)
        elem[nme] = elem_rel_err(x, ref)
        errs[nme] = cond_rel_err(x, ref, r["cond_" + nme], 2) if nme in PATHS else plain[nme]
    extra = ""
    if state:
        x = (g["dm0"] if heads is None else gather_heads(g["dm0"], heads)).reshape(-1, 1)
        e_ref = slice_rel_err(x, r["dm0"].reshape(-1, 1), 1)
        e_con = dm0_consistency(g, C0, n0, heads)
        extra = f"; dm0 consistency {e_con:.1e} (tol {DM0_CONSISTENCY:g}), vs oracle {e_ref:.1e}"
        errs["dm0 consistency"] = e_con / DM0_CONSISTENCY * tol
    log(f"  {label}: " + " ".join(f"{k} {v:.1e}" for k, v in errs.items()
                                  if k != "dm0 consistency") + f" (tol {tol:g})" + extra)
    log("    plain normwise: " + " ".join(f"{k} {v:.1e}" for k, v in plain.items() if k in PATHS)
        + "; elementwise: " + " ".join(f"{k} {v:.1e}" for k, v in elem.items()))
    bad = {k: v for k, v in errs.items() if not v < tol}
    assert not bad, bad


CASES = [
    # label, dtype, B, H, T, dqk, dv, chunk, fgate, o, o dtype, state, dstate
    ("fp32 d16 chunk 16", torch.float32, 1, 2, 64, 16, 16, 16, "sigmoid", True, torch.float32, True, True),
    ("fp32 d32/48 chunk 32 exp gate", torch.float32, 1, 2, 96, 32, 48, 32, "exp", True, torch.float32, False, True),
    ("fp32 d64/32 no o, zero state", torch.float32, 2, 1, 64, 64, 32, 16, "sigmoid", False, None, False, False),
    ("bf16 d128 chunk 32", torch.bfloat16, 1, 2, 256, 128, 128, 32, "sigmoid", True, torch.float32, True, True),
    ("bf16 d256 chunk 32 bf16 o", torch.bfloat16, 1, 2, 256, 256, 256, 32, "sigmoid", True, torch.bfloat16, True, True),
    ("bf16 d256/512 chunk 16", torch.bfloat16, 1, 1, 128, 256, 512, 16, "sigmoid", True, torch.float32, True, False),
    # chunk 64: the reverse pass on MFMA (bf16 operands, float32 accumulation)
    ("bf16 d64 chunk 64", torch.bfloat16, 1, 2, 256, 64, 64, 64, "sigmoid", True, torch.float32, True, True),
    ("bf16 d128/192 chunk 64 exp gate bf16 o", torch.bfloat16, 2, 1, 192, 128, 192, 64, "exp", True, torch.bfloat16, False, True),
    ("bf16 d256 chunk 64 no o", torch.bfloat16, 1, 2, 256, 256, 256, 64, "sigmoid", False, None, True, False),
    ("bf16 d256/128 chunk 64 single chunk", torch.bfloat16, 1, 3, 64, 256, 128, 64, "sigmoid", True, torch.float32, True, True),
    ("bf16 d256/512 chunk 64 eight column blocks", torch.bfloat16, 1, 1, 128, 256, 512, 64, "sigmoid", True, torch.float32, True, True),
    # one column block: dv's two terms partly cancel here, which exposed the
    # bf16 rounding of the carried dC in the dv product (now a hi/lo pair)
    ("bf16 d128/64 chunk 64 one column block", torch.bfloat16, 2, 1, 128, 128, 64, 64, "sigmoid", True, torch.float32, True, True),
    # T not a multiple of the chunk: the pass runs on copies padded with
    # tokens that keep the memory unchanged
    ("ragged fp32 d32/48 chunk 16 T=37", torch.float32, 1, 2, 37, 32, 48, 16, "sigmoid", True, torch.float32, True, True),
    ("ragged fp32 chunk 32 exp gate no o T=50", torch.float32, 2, 1, 50, 64, 32, 32, "exp", False, None, True, True),
    ("ragged bf16 d256/128 chunk 64 T=150", torch.bfloat16, 1, 2, 150, 256, 128, 64, "sigmoid", True, torch.float32, True, True),
    ("ragged bf16 d128/192 chunk 64 exp gate bf16 o T=100", torch.bfloat16, 1, 1, 100, 128, 192, 64, "exp", True, torch.bfloat16, False, True),
    ("ragged bf16 d64 chunk 64 T=9", torch.bfloat16, 1, 2, 9, 64, 64, 64, "sigmoid", True, torch.float32, True, True),
    ("ragged bf16 d64 chunk 64 T=1", torch.bfloat16, 1, 1, 1, 64, 64, 64, "sigmoid", True, torch.float32, True, True),
    # exponential forget gate without o-gate over 9 heads: the long memory
    # keeps the denominator on its active branch, where the gradient's memory
    # and normalizer paths cancel most
    ("bf16 d128/64 chunk 64 one column block exp gate no o 9 heads", torch.bfloat16, 3, 3, 128, 128, 64, 64, "exp", False, None, True, True),
    ("bf16 d128/64 chunk 64 exp gate no o 9 heads T=256", torch.bfloat16, 1, 9, 256, 128, 64, 64, "exp", False, None, True, True),
    ("bf16 d64 chunk 32 exp gate no o 9 heads", torch.bfloat16, 1, 9, 128, 64, 64, 32, "exp", False, None, True, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bwd_parity(case):
    label, dt, B, H, T, dqk, dv, chunk, fgate, o, odt, state, dstate = case
    log(f"bwd {label}")
    f_dist = (4.0, 2.0) if fgate == "sigmoid" else (-0.05, 0.1)
    inp, gin = make_inputs(1, dt, B, H, T, dqk, dv, o=o, state=state, dstate=dstate, f_dist=f_dist)
    h = oracle_h(inp, fgate, odt)
    g = run_gpu(inp, gin, chunk, fgate, odt, h)
    r = run_oracle(inp, gin, fgate, odt, h)
    compare(g, r, TOL_F32 if dt == torch.float32 else TOL_BF16, label, state, C0=inp["C0"],
            n0=inp["n0"])


def test_bwd_chunk_independent():
    """Chunk 16 and chunk 32 give the same gradients (float32 inputs)."""
    inp, gin = make_inputs(3, torch.float32, 1, 2, 128, 32, 32)
    h = oracle_h(inp, "sigmoid", torch.float32)
    g16 = run_gpu(inp, gin, 16, "sigmoid", torch.float32, h)
    g32 = run_gpu(inp, gin, 32, "sigmoid", torch.float32, h)
    for k in ("dq", "dk", "dv", "di", "df", "do", "dC0", "dn0"):
        assert slice_rel_err(g16[k], g32[k]) < 1e-5, k


@pytest.fixture(scope="module")
def d256_case():
    """The measured workload's shape (B=8, H=8, T=8192, d=256, bf16, f32 o-gate,
    random state in, final-state gradient): h of every head from the oracle's
    forward, and the oracle's gradients of two sampled heads."""
    log("bwd d256 T8192 full: inputs")
    inp, gin = make_inputs(2, torch.bfloat16, 8, 8, 8192, 256, 256)
    log("bwd d256 T8192 full: oracle forward (h of all heads)")
    h = oracle_h(inp, "sigmoid", torch.float32)
    heads = sample_heads(8, 8, 2, seed=5)
    log(f"bwd d256 T8192 full: oracle backward on heads {heads}")
    r = run_oracle(inp, gin, "sigmoid", torch.float32, gather_heads(h, heads), heads=heads)
    return inp, gin, h, heads, r


@pytest.mark.parametrize("chunk", [32, 64])
def test_bwd_d256_T8192_sampled_heads(d256_case, chunk):
    """The GPU computes every head of the measured workload, the oracle two
    sampled heads (chunk 32: the float32 reverse pass; chunk 64: MFMA)."""
    inp, gin, h, heads, r = d256_case
    log(f"bwd d256 T8192 full: GPU chunk {chunk}")
    g = run_gpu(inp, gin, chunk, "sigmoid", torch.float32, h)
    compare(g, r, TOL_BF16, f"d256 T8192 sampled chunk {chunk}", True, heads=heads, C0=inp["C0"],
            n0=inp["n0"])


def test_bwd_graph_capture_replays():
    """The chunk-64 backward captured into a HIP graph (its beta pass forks
    onto the library's side stream and joins back inside the capture): three
    replays, with eager work and a synchronization between them, each equal
    bit for bit to the eager call (the passes are deterministic)."""
    M = _M()
    inp, gin = make_inputs(11, torch.bfloat16, 2, 2, 256, 128, 128)
    h = oracle_h(inp, "sigmoid", torch.float32).to("cuda")
    d = to_dev(inp)
    gd = to_dev(gin)
    args = (d["q"], d["k"], d["v"], d["i_pre"], d["f_pre"], d["o_pre"], d["C0"], d["n0"], d["m0"],
            h, gd["dh"], gd["dC1"], gd["dn1"])
    eager = M.mlstm_bwd_chunkwise(*args, chunk=64)
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in eager.items() if v is not None}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up on another stream before capturing
        M.mlstm_bwd_chunkwise(*args, chunk=64)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = M.mlstm_bwd_chunkwise(*args, chunk=64)
    for rep in range(3):
        for v in out.values():
            if v is not None:
                v.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in eager.items():
            assert torch.equal(out[k], v), (rep, k)
