"""GPU parity of the parallel (quadratic) form (mlstm_fwd_parallel) against the
fp64 oracle."""
from __future__ import annotations

import pytest
import torch

import workloads
from helpers import TOL_BF16, TOL_F32, has_gpu, log, slice_rel_err, state_errors, to_dev
from test_gpu_chunkwise import run_oracle

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]


def run_parallel(inp, fgate="sigmoid"):
    import mlstm_matrix_memory_chunkwise_amd as M
    d = to_dev(inp)
    h, (C1, n1, m1) = M.mlstm_fwd_parallel(d["q"], d["k"], d["v"], d["i_pre"], d["f_pre"],
                                           d["o_pre"], d["C0"], d["n0"], d["m0"], fgate=fgate)
    torch.cuda.synchronize()
    return h.cpu(), C1.cpu(), n1.cpu(), m1.cpu()


def _cmp(inp, tol, label, fgate="sigmoid"):
    h, C1, n1, m1 = run_parallel(inp, fgate)
    hr, Cr, nr, mr = run_oracle(inp, fgate=fgate)
    e_h = slice_rel_err(h, hr)
    eC, en, em = state_errors(C1, n1, m1, Cr, nr, mr)
    log(f"  {label}: h {e_h:.2e} C {eC:.2e} n {en:.2e} m {em:.2e}")
    assert max(e_h, eC, en, em) < tol


def test_parallel_tiny_fp32():
    log("parallel tiny fp32")
    _cmp(workloads.make_chunkwise_inputs(workloads.CONFIGS["tiny_fp32"]), TOL_F32, "tiny fp32")


def test_parallel_d128_T2048():
    log("parallel d128 T2048")
    _cmp(workloads.make_chunkwise_inputs(workloads.CONFIGS["d128_T2048"]), TOL_BF16, "d128 T2048")


def test_parallel_state_ragged_T():
    """Random initial state, the d256 T8192 distributions, T not a multiple of the 64-token
    blocks, asymmetric dims."""
    cfg = workloads.Config("par", 5, "bf16", 2, 2, 300, 64, 96, (), (-2.0, 3.0), (4.0, 2.0),
                           (0.0, 1.0), True)
    log("parallel ragged T with state")
    _cmp(workloads.make_chunkwise_inputs(cfg), TOL_BF16, "ragged")


def test_parallel_fp32_exp_gate():
    cfg = workloads.Config("par32", 6, "f32", 1, 3, 130, 32, 16, (), (0.0, 1.0), (-0.05, 0.1),
                           None, True)
    log("parallel fp32 exp gate")
    _cmp(workloads.make_chunkwise_inputs(cfg), TOL_F32, "fp32 exp", fgate="exp")


def test_parallel_matches_chunkwise():
    import mlstm_matrix_memory_chunkwise_amd as M
    cfg = workloads.CONFIGS["d128_T2048"]
    inp = workloads.make_chunkwise_inputs(cfg, B=1, H=4, T=512)
    d = to_dev(inp)
    hp, _ = M.mlstm_fwd_parallel(d["q"], d["k"], d["v"], d["i_pre"], d["f_pre"], d["o_pre"])
    hc, _ = M.mlstm_fwd_chunkwise(d["q"], d["k"], d["v"], d["i_pre"], d["f_pre"], d["o_pre"],
                                  chunk=64)
    torch.cuda.synchronize()
    assert slice_rel_err(hp.cpu(), hc.cpu()) < TOL_BF16


# The bf16 MFMA output kernel (d_qk 64/128/256, d_v a multiple of 64): ragged
# T (the last query and key blocks partial), the initial-state readout, every
# o-gate form, both forget gates, input-gate spikes, several column blocks,
# T below one block and T = 1.  A T that is a multiple of 64 takes the final
# state from the state-only chunk pass, any other T from the per-element
# kernel.
MFMA_CASES = [
    # label, B, H, T, d_qk, d_v, random state, o-gate dtype, fgate, i dist
    ("d64 dv64 T300 state", 2, 2, 300, 64, 64, True, "f32", "sigmoid", (0.0, 1.0)),
    ("d128 dv128 T1000 state bf16-o", 1, 3, 1000, 128, 128, True, "bf16", "sigmoid", (-2.0, 3.0)),
    ("d256 dv192 T512 state", 1, 2, 512, 256, 192, True, "f32", "sigmoid", (-2.0, 3.0)),
    ("d256 dv64 T640 no o-gate exp gate", 1, 2, 640, 256, 64, False, None, "exp", (0.0, 1.0)),
    ("d128 dv64 T37 (one partial block)", 2, 1, 37, 128, 64, True, "f32", "sigmoid", (0.0, 1.0)),
    ("d64 dv64 T1", 1, 2, 1, 64, 64, True, "f32", "sigmoid", (0.0, 1.0)),
    ("d256 dv128 T1024 input-gate spikes", 1, 2, 1024, 256, 128, True, "f32", "sigmoid", (0.0, 15.0)),
]


@pytest.mark.parametrize("case", MFMA_CASES, ids=[c[0] for c in MFMA_CASES])
def test_parallel_mfma_cases(case):
    label, B, H, T, dqk, dv, state, odt, fgate, idist = case
    fdist = (-0.05, 0.1) if fgate == "exp" else (3.0, 1.0)
    cfg = workloads.Config("parm", 7, "bf16", B, H, T, dqk, dv, (), idist, fdist,
                           None if odt is None else (0.0, 1.0), state, fgate)
    inp = workloads.make_chunkwise_inputs(cfg)
    if odt == "bf16":
        inp["o_pre"] = inp["o_pre"].to(torch.bfloat16)
    log(f"parallel MFMA {label}")
    _cmp(inp, TOL_BF16, label, fgate=fgate)
