"""GPU parity of the block operations (mlstm_groupnorm_ogate,
mlstm_causal_conv1d) against the fp64 oracle (oracle/block_ops.py, pinned in
test_oracle_block.py).

Both kernels compute in float32 from exactly representable inputs and round
the output once, so float32 results are held to 1e-4 and bf16 results to the
rounding floor 2^-8 plus that (normwise per slice)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from oracle import block_ops
from helpers import TOL_BF16, TOL_BF16_ROUNDED, TOL_F32, has_gpu, log, slice_rel_err

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]


def _M():
    import mlstm_matrix_memory_chunkwise_amd as M
    return M


def _tol(dt):
    return TOL_F32 if dt == torch.float32 else TOL_BF16_ROUNDED


# ------------------------------------------------------------------ GroupNorm

def gn_inputs(seed, B, H, T, dv, hdt, odt, o=True, affine=True):
    g = torch.Generator().manual_seed(seed)
    h = (torch.randn(B, H, T, dv, generator=g) * 1.5 + 0.2).to(hdt)
    op = torch.randn(B, H, T, dv, generator=g).to(odt) if o else None
    gamma = torch.randn(H, dv, generator=g) * 0.5 + 1.0 if affine else None
    beta = torch.randn(H, dv, generator=g) * 0.5 if affine else None
    return h, op, gamma, beta


GN_CASES = [
    # label, B, H, T, d_v, h dtype, o dtype, o, affine, eps
    ("fp32 d64", 2, 3, 17, 64, torch.float32, torch.float32, True, True, 1e-5),
    ("bf16 d256 f32 o", 2, 2, 33, 256, torch.bfloat16, torch.float32, True, True, 1e-5),
    ("bf16 d128 bf16 o", 1, 4, 9, 128, torch.bfloat16, torch.bfloat16, True, True, 1e-3),
    ("fp32 d20 no o, no affine", 1, 2, 5, 20, torch.float32, torch.float32, False, False, 0.1),
    ("fp32 d1024", 1, 1, 7, 1024, torch.float32, torch.float32, True, True, 1e-5),
    ("bf16 d4", 3, 1, 5, 4, torch.bfloat16, torch.float32, True, False, 1e-5),
]


@pytest.mark.parametrize("case", GN_CASES, ids=[c[0] for c in GN_CASES])
def test_groupnorm_parity(case):
    label, B, H, T, dv, hdt, odt, o, affine, eps = case
    log(f"groupnorm {label}")
    h, op, gamma, beta = gn_inputs(1, B, H, T, dv, hdt, odt, o, affine)
    dev = lambda t: None if t is None else t.cuda()  # noqa: E731
    y = _M().mlstm_groupnorm_ogate(dev(h), dev(op), dev(gamma), dev(beta), eps)
    torch.cuda.synchronize()
    r = block_ops.groupnorm_ogate(h, op, gamma, beta, eps)
    e = slice_rel_err(y.cpu(), r, 2)
    log(f"  {label}: {e:.2e}")
    assert e < _tol(hdt)


def test_groupnorm_in_place():
    h, op, gamma, beta = gn_inputs(2, 2, 2, 16, 256, torch.bfloat16, torch.float32)
    r = block_ops.groupnorm_ogate(h, op, gamma, beta, 1e-5)
    hd = h.cuda()
    y = _M().mlstm_groupnorm_ogate(hd, op.cuda(), gamma.cuda(), beta.cuda(), 1e-5, out=hd)
    torch.cuda.synchronize()
    assert y.data_ptr() == hd.data_ptr()
    assert slice_rel_err(hd.cpu(), r, 2) < TOL_BF16_ROUNDED


def test_groupnorm_full_size_sampled():
    """The cell output shape of the measured workload (B=8, H=8, T=8192,
    d_v=256, bf16 h, f32 o-gate): every row on the GPU, two heads compared."""
    B, H, T, dv = 8, 8, 8192, 256
    log("groupnorm full size")
    h, op, gamma, beta = gn_inputs(3, B, H, T, dv, torch.bfloat16, torch.float32)
    y = _M().mlstm_groupnorm_ogate(h.cuda(), op.cuda(), gamma.cuda(), beta.cuda(), 1e-5).cpu()
    for b, hd in ((0, 0), (7, 5)):
        r = block_ops.groupnorm_ogate(h[b:b + 1], op[b:b + 1], gamma, beta, 1e-5)[:, hd:hd + 1]
        assert slice_rel_err(y[b:b + 1, hd:hd + 1], r, 2) < TOL_BF16_ROUNDED


def test_cell_then_groupnorm_pipeline():
    """The block order: cell without its own gate (o_pre None), then the
    normalization with the gate, against the oracle's cell and normalization."""
    M = _M()
    g = torch.Generator().manual_seed(4)
    B, H, T, d = 1, 2, 256, 128
    q = torch.randn(B, H, T, d, generator=g).to(torch.bfloat16)
    k = (torch.randn(B, H, T, d, generator=g) / d ** 0.5).to(torch.bfloat16)
    v = torch.randn(B, H, T, d, generator=g).to(torch.bfloat16)
    i_pre = torch.randn(B, H, T, generator=g) * 3 - 2
    f_pre = torch.randn(B, H, T, generator=g) * 2 + 4
    o_pre = torch.randn(B, H, T, d, generator=g)
    gamma = torch.randn(H, d, generator=g) * 0.5 + 1
    beta = torch.randn(H, d, generator=g) * 0.5
    h, _ = M.mlstm_fwd_chunkwise(q.cuda(), k.cuda(), v.cuda(), i_pre.cuda(), f_pre.cuda(), None,
                                 chunk=64)
    y = M.mlstm_groupnorm_ogate(h, o_pre.cuda(), gamma.cuda(), beta.cuda(), 1e-5).cpu()
    hr, _, _, _ = oracle.recurrent(q, k, v, i_pre, f_pre, None, None, None, None)
    r = block_ops.groupnorm_ogate(hr, o_pre, gamma, beta, 1e-5)
    e = slice_rel_err(y, r, 2)
    log(f"  cell + groupnorm: {e:.2e}")
    assert e < TOL_BF16


# ------------------------------------------------------------------ causal conv

def conv_inputs(seed, B, T, C, K, dt, bias=True, state=True):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(B, T, C, generator=g).to(dt)
    w = torch.randn(C, K, generator=g) / K ** 0.5
    b = torch.randn(C, generator=g) if bias else None
    s = torch.randn(B, K - 1, C, generator=g) if state else None
    return x, w, b, s


CONV_CASES = [
    # label, B, T, C, K, dtype, bias, state
    ("fp32 K4 ragged T", 2, 100, 12, 4, torch.float32, True, True),
    ("bf16 K4", 2, 130, 64, 4, torch.bfloat16, True, False),
    ("bf16 K1", 1, 70, 16, 1, torch.bfloat16, False, False),
    ("bf16 K8 state", 3, 65, 24, 8, torch.bfloat16, True, True),
    ("fp32 K3 T2 = K-1", 2, 2, 8, 3, torch.float32, False, True),
    ("fp32 K4 T1 decode", 4, 1, 32, 4, torch.float32, True, True),
]


def _conv_check(x, w, b, s, y, st, label):
    r, rs = block_ops.causal_conv1d(x, w, b, s)
    e = slice_rel_err(y.cpu(), r, 1)
    es = slice_rel_err(st.cpu(), rs, 1) if rs.size else 0.0
    log(f"  {label}: y {e:.2e} state {es:.2e}")
    assert e < _tol(x.dtype)
    assert es == 0.0   # the carried window is a copy of inputs


@pytest.mark.parametrize("case", CONV_CASES, ids=[c[0] for c in CONV_CASES])
def test_conv_parity(case):
    label, B, T, C, K, dt, bias, state = case
    log(f"conv {label}")
    x, w, b, s = conv_inputs(1, B, T, C, K, dt, bias, state)
    dev = lambda t: None if t is None else t.cuda()  # noqa: E731
    y, st = _M().mlstm_causal_conv1d(dev(x), dev(w), dev(b), dev(s))
    torch.cuda.synchronize()
    _conv_check(x, w, b, s, y, st, label)


def test_conv_segments_chain():
    """Three segments with the carried window equal one pass (bitwise: the
    same float32 operations in the same order)."""
    M = _M()
    x, w, b, _ = conv_inputs(2, 2, 300, 64, 4, torch.bfloat16)
    xd, wd, bd = x.cuda(), w.cuda(), b.cuda()
    y_full, s_full = M.mlstm_causal_conv1d(xd, wd, bd)
    st = None
    parts = []
    for lo, hi in ((0, 1), (1, 129), (129, 300)):
        yp, st = M.mlstm_causal_conv1d(xd[:, lo:hi].contiguous(), wd, bd, st)
        parts.append(yp)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(parts, 1), y_full)
    assert torch.equal(st, s_full)


def test_conv_full_size():
    """The q/k path of the measured workload: x [B=8, T=8192, C=H*d=2048] bf16,
    K=4, bias and a carried window: every output against the oracle."""
    B, T, C, K = 8, 8192, 2048, 4
    log("conv full size")
    x, w, b, s = conv_inputs(3, B, T, C, K, torch.bfloat16)
    y, st = _M().mlstm_causal_conv1d(x.cuda(), w.cuda(), b.cuda(), s.cuda())
    torch.cuda.synchronize()
    _conv_check(x, w, b, s, y, st, "full size")
