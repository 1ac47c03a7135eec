"""GPU parity of the decode step (mlstm_step) against the fp64 oracle.

The step computes in float32 throughout (bf16 inputs are widened exactly), so
the float32 state is held to the float32 bound (1e-4) for both dtypes, and a
bf16 h to the bf16 rounding floor 2^-8 (plus 1e-4): both far tighter than the
2e-2 allowed for bf16 inputs.
"""
from __future__ import annotations

import pytest
import torch

import oracle
import workloads
from helpers import (TOL_BF16_ROUNDED, TOL_F32, f64, gather_heads, has_gpu, log, sample_heads, slice_rel_err,
                     state_errors, to_dev)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]


def _lib():
    import mlstm_matrix_memory_chunkwise_amd as M
    return M


def _small_inputs(dtype, B, H, dqk, dv, steps, seed, with_o=True, f_dist=(3.0, 1.0)):
    cfg = workloads.Config("small", 9, dtype, B, H, steps, dqk, dv, (), (0.0, 1.0), f_dist,
                           (0.0, 1.0), True, kind="step")
    return workloads.make_step_inputs(cfg, with_o=with_o, seed=seed)


def _run(inp, steps, *, inplace, fgate="sigmoid", o_bf16=False):
    M = _lib()
    d = to_dev(inp)
    C, n, m = d["C0"].clone(), d["n0"].clone(), d["m0"].clone()
    hs = []
    for s in range(steps):
        o = None if d["o_pre"] is None else d["o_pre"][s]
        if o is not None and o_bf16:
            o = o.to(torch.bfloat16)
        h, (C1, n1, m1) = M.mlstm_step(d["q"][s], d["k"][s], d["v"][s], d["i_pre"][s],
                                       d["f_pre"][s], o, C, n, m, fgate=fgate, inplace=inplace)
        if not inplace:
            C, n, m = C1, n1, m1
        hs.append(h)
    torch.cuda.synchronize()
    return torch.stack(hs).cpu(), C.cpu(), n.cpu(), m.cpu()


def _oracle(inp, steps, fgate="sigmoid", o_round_bf16=False):
    C, n, m = f64(inp["C0"]), f64(inp["n0"]), f64(inp["m0"])
    hs = []
    for s in range(steps):
        o = inp["o_pre"]
        if o is not None:
            o = o[s].to(torch.bfloat16) if o_round_bf16 else o[s]
        h, C, n, m = oracle.step(inp["q"][s], inp["k"][s], inp["v"][s], inp["i_pre"][s],
                                 inp["f_pre"][s], o, C, n, m, fgate=fgate)
        hs.append(h)
    import numpy as np
    return np.stack(hs), C, n, m


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("inplace", [False, True])
def test_step_small(dtype, inplace):
    log(f"step small dtype={dtype} inplace={inplace}")
    inp = _small_inputs(dtype, 2, 3, 32, 48, 12, seed=11)
    h, C, n, m = _run(inp, 12, inplace=inplace)
    hr, Cr, nr, mr = _oracle(inp, 12)
    e_h = slice_rel_err(h.permute(1, 2, 0, 3), torch.from_numpy(hr).permute(1, 2, 0, 3))
    eC, en, em = state_errors(C, n, m, Cr, nr, mr)
    log(f"  h {e_h:.2e} C {eC:.2e} n {en:.2e} m {em:.2e}")
    assert e_h < (TOL_F32 if dtype == "f32" else TOL_BF16_ROUNDED)
    assert max(eC, en, em) < TOL_F32


@pytest.mark.parametrize("dqk,dv", [(16, 16), (64, 80), (144, 32), (512, 512)])
def test_step_shapes(dqk, dv):
    log(f"step shapes dqk={dqk} dv={dv}")
    inp = _small_inputs("bf16", 3, 2, dqk, dv, 5, seed=dqk + dv)
    h, C, n, m = _run(inp, 5, inplace=True)
    hr, Cr, nr, mr = _oracle(inp, 5)
    e_h = slice_rel_err(h.permute(1, 2, 0, 3), torch.from_numpy(hr).permute(1, 2, 0, 3))
    eC, en, em = state_errors(C, n, m, Cr, nr, mr)
    assert e_h < TOL_BF16_ROUNDED
    assert max(eC, en, em) < TOL_F32


def test_step_exp_gate_no_output_gate():
    log("step exp gate, no o")
    inp = _small_inputs("f32", 2, 2, 32, 32, 10, seed=5, with_o=False, f_dist=(-0.1, 0.3))
    h, C, n, m = _run(inp, 10, inplace=False, fgate="exp")
    hr, Cr, nr, mr = _oracle(inp, 10, fgate="exp")
    e_h = slice_rel_err(h.permute(1, 2, 0, 3), torch.from_numpy(hr).permute(1, 2, 0, 3))
    eC, en, em = state_errors(C, n, m, Cr, nr, mr)
    assert max(e_h, eC, en, em) < TOL_F32


def test_step_bf16_output_gate():
    log("step bf16 o")
    inp = _small_inputs("bf16", 2, 2, 32, 64, 6, seed=6)
    h, C, n, m = _run(inp, 6, inplace=True, o_bf16=True)
    hr, Cr, nr, mr = _oracle(inp, 6, o_round_bf16=True)
    e_h = slice_rel_err(h.permute(1, 2, 0, 3), torch.from_numpy(hr).permute(1, 2, 0, 3))
    assert e_h < TOL_BF16_ROUNDED


def test_step_d512_full_sampled_heads():
    """The full decode workload (B=128, H=8, d=512, 256 consecutive in-place
    steps, fp32 o-gate) on the GPU; the oracle follows 6 sampled heads."""
    cfg = workloads.CONFIGS["step_d512"]
    log("step d512 full: generating inputs")
    inp = workloads.make_step_inputs(cfg)
    heads = sample_heads(cfg.B, cfg.H, 6, seed=3)
    M = _lib()
    d = to_dev(inp)
    C, n, m = d["C0"], d["n0"], d["m0"]
    hs = []
    log("step d512 full: 256 GPU steps")
    for s in range(cfg.T):
        h, _ = M.mlstm_step(d["q"][s], d["k"][s], d["v"][s], d["i_pre"][s], d["f_pre"][s],
                            d["o_pre"][s], C, n, m, inplace=True)
        hs.append(torch.stack([h[b, hh] for (b, hh) in heads]))
    torch.cuda.synchronize()
    h_gpu = torch.stack(hs).cpu()                       # [S, N, dv]
    C_gpu = gather_heads(C, heads).cpu()
    n_gpu = gather_heads(n, heads).cpu()
    m_gpu = gather_heads(m, heads).cpu()
    del d, C, n, m
    log("step d512 full: oracle on sampled heads")
    sub = {k: (None if v is None else torch.stack([v[:, b, hh] for (b, hh) in heads], dim=1).unsqueeze(1))
           for k, v in inp.items() if k in ("q", "k", "v", "i_pre", "f_pre", "o_pre")}
    sub["C0"] = gather_heads(inp["C0"], heads)
    sub["n0"] = gather_heads(inp["n0"], heads)
    sub["m0"] = gather_heads(inp["m0"], heads)
    hr, Cr, nr, mr = _oracle(sub, cfg.T)                # hr [S, 1, N, dv]
    e_h = slice_rel_err(h_gpu.permute(1, 0, 2).unsqueeze(0),
                        torch.from_numpy(hr[:, 0]).permute(1, 0, 2).unsqueeze(0))
    eC, en, em = state_errors(C_gpu, n_gpu, m_gpu, Cr, nr, mr)
    log(f"  step d512: h {e_h:.2e} C {eC:.2e} n {en:.2e} m {em:.2e}")
    assert e_h < TOL_BF16_ROUNDED
    assert max(eC, en, em) < TOL_F32
