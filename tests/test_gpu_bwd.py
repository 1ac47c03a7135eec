"""GPU parity of the chunkwise backward pass (mlstm_bwd_chunkwise) against the
fp64 gradient oracle (oracle.backward, pinned in test_oracle_bwd.py).

The GPU backward takes the forward output h of the same inputs (as computed
by mlstm_fwd_chunkwise on the GPU); the oracle differentiates its own fp64
forward pass.  Every gradient is compared with the normwise relative error
per (batch, head), at the float32 and bf16 tolerances of the forward."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from helpers import TOL_BF16, TOL_F32, gather_heads, has_gpu, log, sample_heads, slice_rel_err, to_dev

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


def run_gpu(inp, gin, chunk, fgate, o_dtype):
    M = _M()
    d = to_dev(inp)
    gd = to_dev(gin)
    o = None if d["o_pre"] is None else d["o_pre"].to(o_dtype)
    h, _ = M.mlstm_fwd_chunkwise(d["q"], d["k"], d["v"], d["i_pre"], d["f_pre"], o,
                                 d["C0"], d["n0"], d["m0"], chunk=chunk, fgate=fgate)
    g = M.mlstm_bwd_chunkwise(d["q"], d["k"], d["v"], d["i_pre"], d["f_pre"], o,
                              d["C0"], d["n0"], d["m0"], h, gd["dh"], gd["dC1"], gd["dn1"],
                              chunk=chunk, fgate=fgate)
    torch.cuda.synchronize()
    return {k: (None if v is None else v.cpu()) for k, v in g.items()}


def run_oracle(inp, gin, fgate, o_dtype, heads=None):
    sel = (lambda t: t) if heads is None else (lambda t: gather_heads(t, heads))
    x = {k: (None if v is None else sel(v)) for k, v in {**inp, **gin}.items()}
    o = None if x["o_pre"] is None else x["o_pre"].to(o_dtype)
    return oracle.backward(x["q"], x["k"], x["v"], x["i_pre"], x["f_pre"], o, x["C0"], x["n0"],
                           x["m0"], x["dh"], x["dC1"], x["dn1"], fgate=fgate)


def compare(g, r, tol, label, state, heads=None):
    names = ["dq", "dk", "dv", "di", "df"] + (["do"] if r["do"] is not None else [])
    names += ["dC0", "dn0", "dm0"] if state else ["dC0", "dn0"]
    errs = {}
    for nme in names:
        x = g[nme] if heads is None else gather_heads(g[nme], heads)
        lead = 1 if nme == "dm0" else 2
        ref = r[nme]
        if nme == "dm0":
            x = x.reshape(-1, 1)
            ref = ref.reshape(-1, 1)
        errs[nme] = slice_rel_err(x, ref, lead)
    log(f"  {label}: " + " ".join(f"{k} {v:.1e}" for k, v in errs.items()) + f" (tol {tol:g})")
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
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bwd_parity(case):
    label, dt, B, H, T, dqk, dv, chunk, fgate, o, odt, state, dstate = case
    log(f"bwd {label}")
    f_dist = (4.0, 2.0) if fgate == "sigmoid" else (-0.05, 0.1)
    inp, gin = make_inputs(1, dt, B, H, T, dqk, dv, o=o, state=state, dstate=dstate, f_dist=f_dist)
    g = run_gpu(inp, gin, chunk, fgate, odt)
    r = run_oracle(inp, gin, fgate, odt)
    compare(g, r, TOL_F32 if dt == torch.float32 else TOL_BF16, label, state)


def test_bwd_chunk_independent():
    """Chunk 16 and chunk 32 give the same gradients (float32 inputs)."""
    inp, gin = make_inputs(3, torch.float32, 1, 2, 128, 32, 32)
    g16 = run_gpu(inp, gin, 16, "sigmoid", torch.float32)
    g32 = run_gpu(inp, gin, 32, "sigmoid", torch.float32)
    for k in ("dq", "dk", "dv", "di", "df", "do", "dC0", "dn0"):
        assert slice_rel_err(g16[k], g32[k]) < 1e-5, k


@pytest.fixture(scope="module")
def d256_case():
    """The measured workload's shape (B=8, H=8, T=8192, d=256, bf16, f32 o-gate,
    random state in, final-state gradient), with the oracle's gradients of two
    sampled heads."""
    log("bwd d256 T8192 full: inputs")
    inp, gin = make_inputs(2, torch.bfloat16, 8, 8, 8192, 256, 256)
    heads = sample_heads(8, 8, 2, seed=5)
    log(f"bwd d256 T8192 full: oracle on heads {heads}")
    r = run_oracle(inp, gin, "sigmoid", torch.float32, heads=heads)
    return inp, gin, heads, r


@pytest.mark.parametrize("chunk", [32, 64])
def test_bwd_d256_T8192_sampled_heads(d256_case, chunk):
    """The GPU computes every head of the measured workload, the oracle two
    sampled heads (chunk 32: the float32 reverse pass; chunk 64: MFMA)."""
    inp, gin, heads, r = d256_case
    log(f"bwd d256 T8192 full: GPU chunk {chunk}")
    g = run_gpu(inp, gin, chunk, "sigmoid", torch.float32)
    compare(g, r, TOL_BF16, f"d256 T8192 sampled chunk {chunk}", True, heads=heads)
