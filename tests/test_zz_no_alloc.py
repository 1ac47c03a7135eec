"""The entry point that allocates nothing (mlstm_fwd_chunkwise_noalloc),
called through the C ABI, against mlstm_fwd_chunkwise on the same inputs.

The sequences have T not a multiple of the chunk, so the call needs scratch:
the matrix-core kernel leaves its state there and the tail kernel continues
from it.  Two calls in a row, the second smaller, must each equal the
allocating entry point bit for bit (same kernels, same arithmetic) and the
fp64 oracle within the bf16 tolerance."""
from __future__ import annotations

import pytest
import torch

import oracle
import workloads
from helpers import TOL_BF16, has_gpu, log, nan_like, slice_rel_err, state_errors, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]


def _M():
    import mlstm_matrix_memory_chunkwise_amd as M
    return M


CALLS = [
    # B, H, T, d_qk, d_v, chunk (T mod chunk != 0: scratch in use)
    (2, 4, 64 * 5 + 37, 256, 128, 64),
    (1, 3, 64 * 2 + 9, 128, 64, 64),
]


def test_noalloc_matches_allocating_entry_point_twice():
    M = _M()
    for i, (B, H, T, dqk, dv, chunk) in enumerate(CALLS):
        log(f"noalloc call {i}: B={B} H={H} T={T} d_qk={dqk} d_v={dv} chunk={chunk}")
        cfg = workloads.Config("noalloc", 40 + i, "bf16", B, H, T, dqk, dv, (chunk,),
                               (-1.0, 2.0), (3.0, 1.0), (0.0, 1.0), True)
        inp = workloads.make_chunkwise_inputs(cfg)
        need = M.mlstm_fwd_chunkwise_workspace_bytes(M.Problem(B, H, T, dqk, dv, 1, 0, 0, 0),
                                                     chunk)
        assert need > 0
        d = to_dev(inp)
        args = [d[k] for k in ("q", "k", "v", "i_pre", "f_pre", "o_pre", "C0", "n0", "m0")]
        h_a, (C_a, n_a, m_a) = M.mlstm_fwd_chunkwise(*args, chunk=chunk)
        out = nan_like((B, H, T, dv), torch.bfloat16)
        st = (nan_like((B, H, dqk, dv), torch.float32), nan_like((B, H, dqk), torch.float32),
              nan_like((B, H), torch.float32))
        h_b, (C_b, n_b, m_b) = M.mlstm_fwd_chunkwise_noalloc(*args, chunk=chunk, out=out,
                                                             state_out=st)
        torch.cuda.synchronize()
        for name, x, y in (("h", h_b, h_a), ("C1", C_b, C_a), ("n1", n_b, n_a), ("m1", m_b, m_a)):
            assert torch.equal(x, y), f"call {i}: {name} differs from mlstm_fwd_chunkwise"
        hr, Cr, nr, mr = oracle.recurrent(*(inp[k] for k in ("q", "k", "v", "i_pre", "f_pre",
                                                             "o_pre", "C0", "n0", "m0")))
        e_h = slice_rel_err(h_b.cpu(), hr)
        eC, en, em = state_errors(C_b.cpu(), n_b.cpu(), m_b.cpu(), Cr, nr, mr)
        log(f"  noalloc call {i}: bitwise equal; vs oracle h {e_h:.1e} C {eC:.1e} n {en:.1e} "
            f"m {em:.1e}")
        assert max(e_h, eC, en, em) < TOL_BF16


def test_noalloc_split_within_its_scratch():
    """A long sequence with 4 heads of d_v 512: the allocating call splits it
    into 8 segments with more than 64 MiB of workspace; the fixed scratch
    takes the split into 4 segments instead.  Both equal the fp64 oracle on a
    sampled head within the bf16 tolerance, and each other up to rounding."""
    M = _M()
    B, H, T, dqk, dv, chunk = 1, 4, 16384, 256, 512, 64
    need = M.mlstm_fwd_chunkwise_workspace_bytes(M.Problem(B, H, T, dqk, dv, 1, 0, 0, 0), chunk)
    assert need > 64 << 20
    log(f"noalloc split: B={B} H={H} T={T} d_qk={dqk} d_v={dv} chunk={chunk}, workspace {need}")
    cfg = workloads.Config("noalloc_split", 44, "bf16", B, H, T, dqk, dv, (chunk,),
                           (-1.0, 2.0), (3.0, 1.0), (0.0, 1.0), True)
    inp = workloads.make_chunkwise_inputs(cfg)
    d = to_dev(inp)
    args = [d[k] for k in ("q", "k", "v", "i_pre", "f_pre", "o_pre", "C0", "n0", "m0")]
    h_a, (C_a, n_a, m_a) = M.mlstm_fwd_chunkwise(*args, chunk=chunk)
    out = nan_like((B, H, T, dv), torch.bfloat16)
    st = (nan_like((B, H, dqk, dv), torch.float32), nan_like((B, H, dqk), torch.float32),
          nan_like((B, H), torch.float32))
    h_b, (C_b, n_b, m_b) = M.mlstm_fwd_chunkwise_noalloc(*args, chunk=chunk, out=out, state_out=st)
    torch.cuda.synchronize()
    e_h = slice_rel_err(h_b.cpu(), h_a.cpu())
    eC, en, em = state_errors(C_b.cpu(), n_b.cpu(), m_b.cpu(), C_a.cpu(), n_a.cpu(), m_a.cpu())
    log(f"  noalloc vs allocating: h {e_h:.1e} C {eC:.1e} n {en:.1e} m {em:.1e}")
    assert max(e_h, eC, en, em) < TOL_BF16
    hh = 2   # one head against the oracle
    sel = {k: (None if v is None else v[:, hh:hh + 1].contiguous()) for k, v in inp.items()}
    hr, Cr, nr, mr = oracle.recurrent(*(sel[k] for k in ("q", "k", "v", "i_pre", "f_pre", "o_pre",
                                                         "C0", "n0", "m0")))
    e_h = slice_rel_err(h_b[:, hh:hh + 1].cpu(), hr)
    eC, en, em = state_errors(C_b[:, hh:hh + 1].cpu(), n_b[:, hh:hh + 1].cpu(),
                              m_b[:, hh:hh + 1].cpu(), Cr, nr, mr)
    log(f"  noalloc split vs oracle (head {hh}): h {e_h:.1e} C {eC:.1e} n {en:.1e} m {em:.1e}")
    assert max(e_h, eC, en, em) < TOL_BF16
