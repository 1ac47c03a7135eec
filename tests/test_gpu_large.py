"""Problems whose tensors hold more than 2^31 elements: every index past 2^31
must be formed in 64 bits.  The GPU runs the whole problem; the oracle checks
the last heads, whose elements all lie beyond 2^31, and the first head."""
from __future__ import annotations

import pytest
import torch

import oracle
import workloads
from helpers import TOL_BF16, has_gpu, log, slice_rel_err, state_errors

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]


def _M():
    import mlstm_matrix_memory_chunkwise_amd as M
    return M


def test_chunkwise_beyond_2_31_elements():
    B, H, T, d = 1, 1100, 8192, 256       # q, k, v, h: 2.31e9 elements each
    assert B * H * T * d > 2 ** 31
    log(f"large chunkwise B={B} H={H} T={T} d={d}: inputs on the GPU")
    inp = workloads.make_large_device_inputs(B, H, T, d, d, seed=2311, device="cuda")
    log("large chunkwise: GPU")
    h, (C1, n1, m1) = _M().mlstm_fwd_chunkwise(inp["q"], inp["k"], inp["v"], inp["i_pre"],
                                              inp["f_pre"], None, chunk=64)
    torch.cuda.synchronize()
    for heads in (slice(H - 2, H), slice(0, 1)):
        sl = {k: (None if x is None else x[:, heads].cpu()) for k, x in inp.items()}
        log(f"large chunkwise: oracle on heads {heads.start}..{heads.stop - 1}")
        hr, Cr, nr, mr = oracle.recurrent(sl["q"], sl["k"], sl["v"], sl["i_pre"], sl["f_pre"])
        e_h = slice_rel_err(h[:, heads].cpu(), hr)
        eC, en, em = state_errors(C1[:, heads].cpu(), n1[:, heads].cpu(), m1[:, heads].cpu(),
                                  Cr, nr, mr)
        log(f"  heads {heads.start}..{heads.stop - 1}: h {e_h:.2e} C {eC:.2e} n {en:.2e} "
            f"m {em:.2e} (tol {TOL_BF16:g})")
        assert max(e_h, eC, en, em) < TOL_BF16


def test_step_beyond_2_31_state_elements():
    B, H, d = 1025, 8, 512                # C: 2.15e9 elements
    assert B * H * d * d > 2 ** 31
    log(f"large step B={B} H={H} d={d}: inputs on the GPU")
    s = workloads.make_large_device_step(B, H, d, d, seed=2312, device="cuda")
    # the oracle's copies of the last two heads and the first one, before the in-place update
    picks = ((B - 1, slice(H - 2, H)), (0, slice(0, 1)))
    host = [{k: x[b:b + 1, hs].cpu() for k, x in s.items()} for b, hs in picks]
    log("large step: GPU (in place)")
    h, (C, n, m) = _M().mlstm_step(s["q"], s["k"], s["v"], s["i_pre"], s["f_pre"], s["o_pre"],
                                   s["C"], s["n"], s["m"], inplace=True)
    torch.cuda.synchronize()
    for (b, hs), x in zip(picks, host):
        hr, Cr, nr, mr = oracle.step(x["q"], x["k"], x["v"], x["i_pre"], x["f_pre"], x["o_pre"],
                                     x["C"], x["n"], x["m"])
        e_h = slice_rel_err(h[b:b + 1, hs].cpu(), hr)
        eC, en, em = state_errors(C[b:b + 1, hs].cpu(), n[b:b + 1, hs].cpu(), m[b:b + 1, hs].cpu(),
                                  Cr, nr, mr)
        log(f"  batch {b} heads {hs.start}..{hs.stop - 1}: h {e_h:.2e} C {eC:.2e} n {en:.2e} "
            f"m {em:.2e} (tol {TOL_BF16:g})")
        assert max(e_h, eC, en, em) < TOL_BF16


def test_block_ops_beyond_2_31_elements():
    from oracle import block_ops
    from helpers import TOL_BF16_ROUNDED
    M = _M()
    log("large block ops: inputs on the GPU")
    d = workloads.make_large_device_block_inputs(seed=2313, device="cuda")
    # group normalization + output gate over h [1, 1100, 8192, 256]
    assert d["h"].numel() > 2 ** 31
    log("large group normalization: GPU")
    y = M.mlstm_groupnorm_ogate(d["h"], d["o_pre"], d["gamma"], d["beta"])
    torch.cuda.synchronize()
    for hs, ts in ((slice(1098, 1100), slice(8192 - 64, 8192)), (slice(0, 1), slice(0, 64))):
        ref = block_ops.groupnorm_ogate(d["h"][:, hs, ts].cpu(), d["o_pre"][:, hs, ts].cpu(),
                                        d["gamma"][hs].cpu(), d["beta"][hs].cpu())
        e = slice_rel_err(y[:, hs, ts].cpu(), ref, lead=3)
        log(f"  heads {hs.start}..{hs.stop - 1} tokens {ts.start}..{ts.stop - 1}: y {e:.2e} "
            f"(tol {TOL_BF16_ROUNDED:.2e})")
        assert e < TOL_BF16_ROUNDED
    del y
    # causal conv over x [8, 131200, 2048]
    assert d["x"].numel() > 2 ** 31
    log("large causal conv: GPU")
    yc, st = M.mlstm_causal_conv1d(d["x"], d["w"], d["bias"])
    torch.cuda.synchronize()
    K = d["w"].shape[1]
    TX = d["x"].shape[1]
    for b, ts, cs in ((7, slice(TX - 96, TX), slice(2048 - 64, 2048)),
                      (0, slice(0, 96), slice(0, 64))):
        xs = d["x"][b:b + 1, ts, cs].cpu()
        t0 = ts.start
        if t0 >= K - 1:
            state = d["x"][b:b + 1, t0 - K + 1:t0, cs].float().cpu()
        else:
            state = None
        ref, _ = block_ops.causal_conv1d(xs, d["w"][cs].cpu(), d["bias"][cs].cpu(), state)
        e = slice_rel_err(yc[b:b + 1, ts, cs].cpu(), ref, lead=1)
        log(f"  batch {b} tokens {ts.start}..{ts.stop - 1} channels {cs.start}..{cs.stop - 1}: "
            f"y {e:.2e} (tol {TOL_BF16_ROUNDED:.2e})")
        assert e < TOL_BF16_ROUNDED
    ref_state = d["x"][7:8, TX - (K - 1):, 2048 - 64:].float().cpu()
    assert torch.equal(st[7:8, :, 2048 - 64:].cpu(), ref_state)


def test_backward_beyond_2_31_elements():
    """Chunk-64 backward (matrix-core passes) with q, k, v, h, dh of 2.31e9
    elements each and float32 gradients of the same size."""
    B, H, T, d = 1, 1100, 8192, 256
    torch.cuda.empty_cache()
    log(f"large backward B={B} H={H} T={T} d={d}: inputs on the GPU")
    inp = workloads.make_large_device_inputs(B, H, T, d, d, seed=2314, device="cuda")
    gin = workloads.make_large_device_grads(B, H, T, d, d, seed=2315, device="cuda")
    M = _M()
    log("large backward: GPU forward")
    h, _ = M.mlstm_fwd_chunkwise(inp["q"], inp["k"], inp["v"], inp["i_pre"], inp["f_pre"], None,
                                 chunk=64, return_state=False)
    log("large backward: GPU backward")
    g = M.mlstm_bwd_chunkwise(inp["q"], inp["k"], inp["v"], inp["i_pre"], inp["f_pre"], None,
                              None, None, None, h, gin["dh"], gin["dC1"], gin["dn1"], chunk=64)
    torch.cuda.synchronize()
    for heads in (slice(H - 2, H), slice(0, 1)):
        x = {k: (None if t is None else t[:, heads].cpu()) for k, t in {**inp, **gin}.items()}
        log(f"large backward: oracle on heads {heads.start}..{heads.stop - 1}")
        r = oracle.backward(x["q"], x["k"], x["v"], x["i_pre"], x["f_pre"], None, None, None, None,
                            x["dh"], x["dC1"], x["dn1"])
        errs = {n: slice_rel_err(g[n][:, heads].cpu(), r[n]) for n in ("dq", "dk", "dv", "di", "df",
                                                                       "dC0", "dn0")}
        log(f"  heads {heads.start}..{heads.stop - 1}: "
            + " ".join(f"{k} {v:.1e}" for k, v in errs.items()) + f" (tol {TOL_BF16:g})")
        bad = {k: v for k, v in errs.items() if not v < TOL_BF16}
        assert not bad, bad


def test_slstm_beyond_2_31_elements():
    """sLSTM cell with wx of 2.15e9 elements: 256 sequences of 16400 steps."""
    from oracle import slstm
    from helpers import TOL_BF16_ROUNDED
    B, NH, T, DH = 64, 4, 16400, 128
    assert B * NH * T * 4 * DH > 2 ** 31
    torch.cuda.empty_cache()
    log(f"large sLSTM B={B} NH={NH} T={T} DH={DH}: inputs on the GPU")
    d = workloads.make_large_device_slstm(B, NH, T, DH, seed=2316, device="cuda")
    log("large sLSTM: GPU")
    h, _ = _M().mlstm_slstm_fwd(d["wx"], d["R"], return_state=False)
    torch.cuda.synchronize()
    for b, hd in ((B - 1, NH - 1), (0, 0)):
        log(f"large sLSTM: oracle on batch {b} head {hd}")
        wx = d["wx"][b:b + 1, hd:hd + 1].cpu()
        ref, _ = slstm.slstm_forward(wx, d["R"][hd:hd + 1].cpu())
        e = slice_rel_err(h[b:b + 1, hd:hd + 1].cpu(), ref)
        log(f"  batch {b} head {hd}: h {e:.2e} (tol {TOL_BF16_ROUNDED:.2e})")
        assert e < TOL_BF16_ROUNDED


def test_parallel_beyond_2_31_elements():
    """Quadratic (parallel) form with q, k, v, h of 2.15e9 elements each: many
    short heads keep its O(T^2) work small."""
    B, H, T, d = 1, 16400, 512, 256
    assert B * H * T * d > 2 ** 31
    torch.cuda.empty_cache()
    log(f"large parallel B={B} H={H} T={T} d={d}: inputs on the GPU")
    inp = workloads.make_large_device_inputs(B, H, T, d, d, seed=2317, device="cuda")
    log("large parallel: GPU")
    h, (C1, n1, m1) = _M().mlstm_fwd_parallel(inp["q"], inp["k"], inp["v"], inp["i_pre"],
                                             inp["f_pre"])
    torch.cuda.synchronize()
    for heads in (slice(H - 2, H), slice(0, 1)):
        sl = {k: (None if x is None else x[:, heads].cpu()) for k, x in inp.items()}
        hr, Cr, nr, mr = oracle.recurrent(sl["q"], sl["k"], sl["v"], sl["i_pre"], sl["f_pre"])
        e_h = slice_rel_err(h[:, heads].cpu(), hr)
        eC, en, em = state_errors(C1[:, heads].cpu(), n1[:, heads].cpu(), m1[:, heads].cpu(),
                                  Cr, nr, mr)
        log(f"  heads {heads.start}..{heads.stop - 1}: h {e_h:.2e} C {eC:.2e} n {en:.2e} "
            f"m {em:.2e} (tol {TOL_BF16:g})")
        assert max(e_h, eC, en, em) < TOL_BF16
