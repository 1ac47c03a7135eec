"""GPU parity of the sLSTM forward cell (mlstm_slstm_fwd) against the fp64
oracle (oracle/slstm.py, pinned in test_oracle_slstm.py).

The kernel computes in float32 and feeds the float32 h back, so float32
outputs are held to 1e-4 and bf16 outputs (a rounded copy of h, from exactly
representable bf16 inputs) to the rounding floor 2^-8 plus that."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle import slstm
from helpers import TOL_BF16_ROUNDED, TOL_F32, has_gpu, log, slice_rel_err

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]


def _M():
    import mlstm_matrix_memory_chunkwise_amd as M
    return M


def slstm_inputs(seed, B, NH, T, DH, dt, fgate="sigmoid", state=True):
    """i~ ~ N(-1, 1), f~ ~ N(3, 1) (sigmoid gate) or N(-0.05, 0.1) (exp gate),
    z, o~ ~ N(0, 1); R ~ N(0, 0.5 / sqrt(DH)); state c0 ~ N(0, 1),
    n0 ~ U(0.5, 2), m0 ~ N(0, 1), h0 ~ N(0, 0.5)."""
    g = torch.Generator().manual_seed(seed)
    wx = torch.randn(B, NH, T, 4, DH, generator=g)
    wx[:, :, :, 0] = wx[:, :, :, 0] - 1.0
    if fgate == "sigmoid":
        wx[:, :, :, 1] = wx[:, :, :, 1] + 3.0
    else:
        wx[:, :, :, 1] = wx[:, :, :, 1] * 0.1 - 0.05
    wx = wx.to(dt)
    R = torch.randn(NH, 4, DH, DH, generator=g) * (0.5 / math.sqrt(DH))
    st = None
    if state:
        st = dict(c0=torch.randn(B, NH, DH, generator=g),
                  n0=torch.rand(B, NH, DH, generator=g) * 1.5 + 0.5,
                  m0=torch.randn(B, NH, DH, generator=g),
                  h0=torch.randn(B, NH, DH, generator=g) * 0.5)
    return wx, R, st


def run_gpu(wx, R, st, fgate):
    d = {} if st is None else {k: v.cuda() for k, v in st.items()}
    h, fin = _M().mlstm_slstm_fwd(wx.cuda(), R.cuda(), fgate=fgate, **d)
    torch.cuda.synchronize()
    return h.cpu(), tuple(x.cpu() for x in fin)


def _tol(dt):
    return TOL_F32 if dt == torch.float32 else TOL_BF16_ROUNDED


CASES = [
    # label, B, NH, T, DH, dtype, fgate, state
    ("fp32 DH16 ragged T", 2, 2, 37, 16, torch.float32, "sigmoid", True),
    ("fp32 DH32 exp gate zero state", 1, 3, 64, 32, torch.float32, "exp", False),
    ("bf16 DH64", 2, 2, 50, 64, torch.bfloat16, "sigmoid", True),
    ("fp32 DH128 one head", 3, 1, 200, 128, torch.float32, "sigmoid", True),
    ("bf16 DH128 T1", 4, 2, 1, 128, torch.bfloat16, "exp", True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_slstm_parity(case):
    label, B, NH, T, DH, dt, fgate, state = case
    log(f"slstm {label}")
    wx, R, st = slstm_inputs(1, B, NH, T, DH, dt, fgate, state)
    h, (c1, n1, m1, h1) = run_gpu(wx, R, st, fgate)
    hr, (cr, nr, mr, hrT) = slstm.slstm_forward(wx, R, fgate=fgate, **({} if st is None else st))
    e = slice_rel_err(h, hr, 2)
    # the final (c, n) are defined up to the stabilizer shift: compare at the oracle's m
    sc = np.exp(m1.double().numpy() - mr)
    ec = slice_rel_err(c1.double().numpy() * sc, cr, 2)
    en = slice_rel_err(n1.double().numpy() * sc, nr, 2)
    eh = slice_rel_err(h1, hrT, 2)
    log(f"  {label}: h {e:.2e} c {ec:.2e} n {en:.2e} h_T {eh:.2e}")
    assert e < _tol(dt)
    assert max(ec, en, eh) < TOL_F32


def test_slstm_split_resume():
    """Two calls with the carried state equal one call (bitwise)."""
    M = _M()
    wx, R, st = slstm_inputs(2, 2, 2, 41, 64, torch.float32)
    wxd, Rd = wx.cuda(), R.cuda()
    std = {k: v.cuda() for k, v in st.items()}
    h, fin = M.mlstm_slstm_fwd(wxd, Rd, **std)
    ha, fa = M.mlstm_slstm_fwd(wxd[:, :, :17].contiguous(), Rd, **std)
    hb, fb = M.mlstm_slstm_fwd(wxd[:, :, 17:].contiguous(), Rd, *fa)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([ha, hb], 2), h)
    for x, y in zip(fb, fin):
        assert torch.equal(x, y)


def test_slstm_measured_shape_sampled():
    """The measured shape (B=64, NH=4, DH=128, T=4096, bf16 wx and h, sigmoid
    gate, random state): every sequence on the GPU, two batch rows (all their
    heads) against the oracle."""
    B, NH, T, DH = 64, 4, 4096, 128
    log("slstm measured shape: inputs")
    wx, R, st = slstm_inputs(3, B, NH, T, DH, torch.bfloat16)
    h, _ = run_gpu(wx, R, st, "sigmoid")
    for b in (0, 63):
        log(f"slstm measured shape: oracle on b={b}")
        sub = {k: v[b:b + 1] for k, v in st.items()}
        hr, _ = slstm.slstm_forward(wx[b:b + 1], R, **sub)
        e = slice_rel_err(h[b:b + 1], hr, 2)
        log(f"  b={b}: h {e:.2e}")
        assert e < TOL_BF16_ROUNDED
