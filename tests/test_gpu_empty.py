"""Empty inputs on the GPU: T = 0 tokens (or steps) with a state, through
the Python binding.  The final state is the initial one (zeros without it);
the backward passes the memory gradient through, checked against the oracle,
which handles T = 0 by its plain loops."""
from __future__ import annotations

import pytest
import torch

import oracle
from helpers import TOL_F32, has_gpu, log, slice_rel_err

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]


def _M():
    import mlstm_matrix_memory_chunkwise_amd as M
    return M


def _seq(B, H, T, d, dtype, seed, state=True):
    g = torch.Generator().manual_seed(seed)
    x = dict(q=torch.zeros(B, H, T, d, dtype=dtype), k=torch.zeros(B, H, T, d, dtype=dtype),
             v=torch.zeros(B, H, T, d, dtype=dtype), i_pre=torch.zeros(B, H, T),
             f_pre=torch.zeros(B, H, T))
    st = dict(C0=torch.randn(B, H, d, d, generator=g), n0=torch.randn(B, H, d, generator=g),
              m0=torch.randn(B, H, generator=g)) if state else dict(C0=None, n0=None, m0=None)
    return {k: (None if t is None else t.cuda()) for k, t in {**x, **st}.items()}


@pytest.mark.parametrize("form", ["chunkwise", "parallel"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_forward_T0_passes_state(form, dtype):
    log(f"empty forward {form} {dtype}")
    M = _M()
    d = _seq(2, 3, 0, 64, dtype, seed=1)
    fn = M.mlstm_fwd_chunkwise if form == "chunkwise" else M.mlstm_fwd_parallel
    kw = dict(chunk=64) if form == "chunkwise" else {}
    h, (C1, n1, m1) = fn(d["q"], d["k"], d["v"], d["i_pre"], d["f_pre"], None,
                         d["C0"], d["n0"], d["m0"], **kw)
    torch.cuda.synchronize()
    assert h.shape == (2, 3, 0, 64)
    assert torch.equal(C1, d["C0"]) and torch.equal(n1, d["n0"]) and torch.equal(m1, d["m0"])
    # no initial state: the final state is zero
    h, (C1, n1, m1) = fn(d["q"], d["k"], d["v"], d["i_pre"], d["f_pre"], None, **kw)
    torch.cuda.synchronize()
    assert not C1.any() and not n1.any() and not m1.any()


@pytest.mark.parametrize("chunk", [16, 64])
def test_backward_T0_against_oracle(chunk):
    log(f"empty backward chunk {chunk}")
    M = _M()
    d = _seq(2, 3, 0, 64, torch.bfloat16, seed=2)
    g = torch.Generator().manual_seed(3)
    dC1 = torch.randn(2, 3, 64, 64, generator=g).cuda()
    dn1 = torch.randn(2, 3, 64, generator=g).cuda()
    dh = torch.zeros(2, 3, 0, 64, dtype=torch.bfloat16, device="cuda")
    h = torch.zeros_like(dh)
    out = M.mlstm_bwd_chunkwise(d["q"], d["k"], d["v"], d["i_pre"], d["f_pre"], None,
                                d["C0"], d["n0"], d["m0"], h, dh, dC1, dn1, chunk=chunk)
    torch.cuda.synchronize()
    c = {k: (None if t is None else t.cpu()) for k, t in d.items()}
    r = oracle.backward(c["q"], c["k"], c["v"], c["i_pre"], c["f_pre"], None, c["C0"], c["n0"],
                        c["m0"], dh.cpu(), dC1.cpu(), dn1.cpu())
    errs = {n: slice_rel_err(out[n].cpu(), r[n], 1 if n == "dm0" else 2)
            for n in ("dC0", "dn0", "dm0")}
    log("  " + " ".join(f"{k} {v:.1e}" for k, v in errs.items()))
    assert max(errs.values()) < TOL_F32
    assert out["dq"].shape == (2, 3, 0, 64) and out["df"].shape == (2, 3, 0)


def test_slstm_and_conv_T0_pass_state():
    log("empty sLSTM and conv")
    M = _M()
    g = torch.Generator().manual_seed(4)
    B, NH, DH = 2, 2, 32
    wx = torch.zeros(B, NH, 0, 4, DH, device="cuda")
    R = torch.randn(NH, 4, DH, DH, generator=g).cuda()
    st = [torch.randn(B, NH, DH, generator=g).cuda() for _ in range(4)]
    h, (c1, n1, m1, h1) = M.mlstm_slstm_fwd(wx, R, *st)
    torch.cuda.synchronize()
    assert h.shape == (B, NH, 0, DH)
    for a, b in zip((c1, n1, m1, h1), st):
        assert torch.equal(a, b)
    x = torch.zeros(3, 0, 64, dtype=torch.bfloat16, device="cuda")
    w = torch.randn(64, 4, generator=g).cuda()
    s_in = torch.randn(3, 3, 64, generator=g).cuda()
    y, s_out = M.mlstm_causal_conv1d(x, w, None, s_in)
    torch.cuda.synchronize()
    assert y.shape == (3, 0, 64) and torch.equal(s_out, s_in)
    y, s_out = M.mlstm_causal_conv1d(x, w)
    torch.cuda.synchronize()
    assert not s_out.any()
    hn = torch.zeros(2, 2, 0, 64, dtype=torch.bfloat16, device="cuda")
    assert M.mlstm_groupnorm_ogate(hn).shape == hn.shape
