"""Benchmark of the mLSTM forward hot path on one MI355X.

One bench step is one chunkwise forward pass (mlstm_fwd_chunkwise) over the
d=256, T=8192 workload: B=8, H=8, d_qk=d_v=256, bf16 q/k/v, fp32 gates and
o-gate preactivation, random initial state carried in and the final state
written out.  value = tokens/s (B*T tokens per pass).  Also reported on the
same line: the decode step (mlstm_step) on its workload (B=128, H=8, d=512,
256 consecutive in-place steps) as GB/s against 8 TB/s, the chunk-128
variant, the variant without o-gate and the cell followed by the group
normalization pass, the long-context workload (B=1, H=16, T=65536, d_qk=256,
d_v=512, chunk 128), the backward pass, the block operations, the sLSTM
cell, the roofline of the dominant kernel, and the fp64 CPU oracle timed on a
bounded sample of the chunkwise workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--chunk 64]
                       [--skip-cpu] [--skip-step] [--skip-extra] [--skip-long]
       python bench.py --profile-workload   (one chunkwise pass and its
           backward, one decode step, the block operations and a 1 GiB
           copy, for rocprofv3 counter runs; prints nothing)

roofline.traffic is the HBM traffic per launch of the dominant kernel from
the committed counter summary (profiles/hbm_traffic.txt: FETCH_SIZE and
WRITE_SIZE of the kernel, scaled by what the same counters read for a copy of
known size); it is null when the kernel sources changed since the counters
were taken (their SHA-256 is recorded with the counters).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s

METRIC = "mLSTM chunkwise fwd tokens/s + % bf16 MFMA peak; step GB/s % HBM peak (1 GPU)"


def chunk_algorithmic(B, H, T, dqk, dv, L, o_bytes, state_in=True, state_out=True):
    """Algorithmic work of one chunkwise pass.

    flops: bf16 MFMA work per token-head (L+1)(d_qk+d_v) (causal halves of Q K^T
    and P V) + 4 d_qk d_v (readout q^T C and the state update k v^T).
    bytes: q, k, v, h (bf16), gates (2 x fp32), o-gate, plus the state in/out
    (the minimum any implementation must move).
    """
    th = B * H * T
    flops = th * ((L + 1) * (dqk + dv) + 4 * dqk * dv)
    per_tok = (2 * dqk + dv) * 2 + dv * 2 + 8 + dv * o_bytes
    state = B * H * (dqk * dv + dqk + 1) * 4
    byts = th * per_tok + state * (int(state_in) + int(state_out))
    return flops, byts


def bwd_algorithmic(B, H, T, dqk, dv, L, o_bytes):
    """Algorithmic work of one chunkwise backward pass.

    flops per token-head: the causal halves of Q K^T, W K, W^T Q (3 (L+1) d_qk)
    and of R V^T, (D S)^T R (2 (L+1) d_v), plus five d_qk x d_v products: the
    state recomputed forward (K^T V), C~_s r, dC v, dC^T k and the state
    gradient Q^T R (10 d_qk d_v).
    bytes: q, k, v, h, dh (bf16), gates, o-gate in; dq, dk, dv, do (float32),
    di, df out; the state and its gradient in and out once.
    """
    th = B * H * T
    flops = th * (3 * (L + 1) * dqk + 2 * (L + 1) * dv + 10 * dqk * dv)
    per_tok = (2 * dqk + 3 * dv) * 2 + 8 + dv * o_bytes + (2 * dqk + 2 * dv) * 4 + 8
    state = B * H * (dqk * dv + dqk + 1) * 4
    byts = th * per_tok + 4 * state
    return flops, byts


def groupnorm_algorithmic(B, H, T, dv, h_bytes=2, o_bytes=4):
    """Bytes of the group normalization with o-gate: h and o~ in, y out,
    gamma and beta once."""
    return B * H * T * dv * (2 * h_bytes + o_bytes) + 2 * H * dv * 4


def conv_algorithmic(B, T, C, K, x_bytes=2):
    """Bytes of the causal depthwise convolution: x in, y out, weights, bias
    and the carried window in and out once."""
    return 2 * B * T * C * x_bytes + C * (K + 1) * 4 + 2 * B * (K - 1) * C * 4


# sLSTM line: 64 sequences x 4 heads of 128 units fill the 256 CUs with one
# (batch, head) sequence each
SLSTM_SHAPE = dict(B=64, NH=4, T=4096, DH=128)
# MI355X fp32 vector peak without packed FP32: 256 CUs x 64 FMA/clk x 2 flop x
# 2.4 GHz = 78.6 TFLOP/s.  The library is built with packed FP32 off, so the
# 157.3 TFLOP/s datasheet figure (two lanes per FMA) is out of reach.
FP32_VALU_PEAK_TFLOPS = 78.6


def slstm_flops(B, NH, T, DH):
    """The recurrent mat-vec products: 4 gates x DH x DH multiply-adds per
    (sequence, head, step); the gate arithmetic is not counted."""
    return 2 * 4 * DH * DH * B * NH * T


# shapes of the block-operation lines: the cell output of the measured
# workload, and its q/k path before the projections ([B, T, H*d_qk])
GN_SHAPE = dict(B=8, H=8, T=8192, dv=256)
CONV_SHAPE = dict(B=8, T=8192, C=2048, K=4)


def block_inputs(dev, seed=7):
    import torch
    g = torch.Generator(device="cpu").manual_seed(seed)
    B, H, T, dv = GN_SHAPE["B"], GN_SHAPE["H"], GN_SHAPE["T"], GN_SHAPE["dv"]
    gn = dict(h=torch.randn((B, H, T, dv), generator=g).to(torch.bfloat16).to(dev),
              o=torch.randn((B, H, T, dv), generator=g).to(dev),
              gamma=(torch.randn((H, dv), generator=g) * 0.5 + 1).to(dev),
              beta=(torch.randn((H, dv), generator=g) * 0.5).to(dev))
    gn["y"] = torch.empty_like(gn["h"])
    B, T, C, K = CONV_SHAPE["B"], CONV_SHAPE["T"], CONV_SHAPE["C"], CONV_SHAPE["K"]
    cv = dict(x=torch.randn((B, T, C), generator=g).to(torch.bfloat16).to(dev),
              w=(torch.randn((C, K), generator=g) / 2).to(dev),
              b=torch.randn((C,), generator=g).to(dev),
              s=torch.randn((B, K - 1, C), generator=g).to(dev))
    cv["y"] = torch.empty_like(cv["x"])
    return gn, cv


def step_algorithmic(B, H, dqk, dv, qkv_bytes=2, o_bytes=4):
    """Bytes one decode step must move: C~ read + write, n~ read + write, m,
    q, k, v, gates, o-gate, h."""
    BH = B * H
    return BH * (2 * dqk * dv * 4 + 2 * dqk * 4 + 2 * 4 + 2 * dqk * qkv_bytes +
                 dv * qkv_bytes + 8 + dv * o_bytes + dv * qkv_bytes)


# sources whose kernels the HBM counters describe
SETTLE_S = 0.15

KERNEL_SOURCES = {
    "groupnorm": ["block_ops.hip", "common.hpp", "kernels.hpp"],
    "conv": ["block_ops.hip", "common.hpp", "kernels.hpp"],
    "chunkwise": ["chunk_ws.hip", "mfma_util.hpp", "common.hpp", "kernels.hpp"],
    "chunk128": ["chunk_ws128.hip", "mfma_util.hpp", "common.hpp", "kernels.hpp"],
    "step": ["step.hip", "common.hpp", "kernels.hpp"],
    "backward": ["bwd.hip", "bwd_mfma.hip", "mfma_util.hpp", "common.hpp", "kernels.hpp"],
    "long_context": ["chunk_ws128.hip", "chunk_mfma.hip", "chunk_state.hip", "state_gemm.hip", "api.hip",
                     "mfma_util.hpp",
                     "common.hpp", "kernels.hpp"],
    "long_context_4heads": ["chunk_ws128.hip", "chunk_mfma.hip", "chunk_state.hip", "state_gemm.hip",
                            "api.hip", "mfma_util.hpp", "common.hpp", "kernels.hpp"],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")


def kernel_sources_sha(which):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mlstm_matrix_memory_chunkwise_amd", "csrc")
    for f in KERNEL_SOURCES[which]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(which, key=None):
    """Calibrated HBM bytes per launch (or `key`) from profiles/hbm_traffic.txt,
    or None when absent or taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            kv = dict(line.split(":", 1) for line in fh if ":" in line and not line.startswith("#"))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get(f"{which}_sources_sha256") != kernel_sources_sha(which):
        return None
    try:
        return float(kv[key or f"{which}_calibrated_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def profile_workload():
    """One launch of each measured kernel plus a copy of known size."""
    import torch

    import mlstm_matrix_memory_chunkwise_amd as M
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    M.load_library()
    cfg = workloads.CONFIGS["d256_T8192"]
    d = {k: (None if v is None else v.to(dev)) for k, v in workloads.make_chunkwise_inputs(cfg).items()}
    h = torch.empty((cfg.B, cfg.H, cfg.T, cfg.dv), dtype=torch.bfloat16, device=dev)
    M.mlstm_fwd_chunkwise(d["q"], d["k"], d["v"], d["i_pre"], d["f_pre"], d["o_pre"],
                          d["C0"], d["n0"], d["m0"], chunk=64, out=h)
    torch.cuda.synchronize()
    # the same pass at chunk 128
    M.mlstm_fwd_chunkwise(d["q"], d["k"], d["v"], d["i_pre"], d["f_pre"], d["o_pre"],
                          d["C0"], d["n0"], d["m0"], chunk=128, out=h)
    torch.cuda.synchronize()
    # the backward of the same pass (chunk 64), as timed by the bench
    gen = torch.Generator(device="cpu").manual_seed(cfg.seed + 1)
    dh = torch.randn((cfg.B, cfg.H, cfg.T, cfg.dv), generator=gen).to(torch.bfloat16).to(dev)
    dC1 = torch.randn((cfg.B, cfg.H, cfg.dqk, cfg.dv), generator=gen).to(dev)
    dn1 = torch.randn((cfg.B, cfg.H, cfg.dqk), generator=gen).to(dev)
    M.mlstm_bwd_chunkwise(d["q"], d["k"], d["v"], d["i_pre"], d["f_pre"], d["o_pre"],
                          d["C0"], d["n0"], d["m0"], h, dh, dC1, dn1, chunk=64)
    torch.cuda.synchronize()
    del d, h, dh, dC1, dn1
    torch.cuda.empty_cache()
    cfg3 = workloads.CONFIGS["step_d512"]
    s = {k: (None if v is None else v.to(dev)) for k, v in workloads.make_step_inputs(cfg3).items()}
    M.mlstm_step(s["q"][0], s["k"][0], s["v"][0], s["i_pre"][0], s["f_pre"][0], s["o_pre"][0],
                 s["C0"], s["n0"], s["m0"], inplace=True)
    torch.cuda.synchronize()
    del s
    gn, cv = block_inputs(dev)
    M.mlstm_groupnorm_ogate(gn["h"], gn["o"], gn["gamma"], gn["beta"], 1e-5, out=gn["y"])
    M.mlstm_causal_conv1d(cv["x"], cv["w"], cv["b"], cv["s"], out=cv["y"])
    torch.cuda.synchronize()
    del gn, cv
    torch.cuda.empty_cache()
    # the long-context forward (chunk 128, sequence split: the states at the
    # split points, then all segments at once, and the state copies), with
    # its 16 heads (2 segments) and with 4 heads (8 segments)
    cfg4 = workloads.CONFIGS["d256x512_T65536"]
    for heads in (cfg4.H, 4):
        d4 = {k: (None if v is None else v.to(dev))
              for k, v in workloads.make_chunkwise_inputs(cfg4, H=heads).items()}
        h4 = torch.empty((cfg4.B, heads, cfg4.T, cfg4.dv), dtype=torch.bfloat16, device=dev)
        M.mlstm_fwd_chunkwise(d4["q"], d4["k"], d4["v"], d4["i_pre"], d4["f_pre"], d4["o_pre"],
                              chunk=cfg4.chunks[0], out=h4)
        torch.cuda.synchronize()
        del d4, h4
        torch.cuda.empty_cache()
    x = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
    y = torch.empty_like(x)
    y.copy_(x)
    torch.cuda.synchronize()


def parallel_flops(B, H, T, dqk, dv):
    """Algorithmic flops of the parallel form's outputs: per head and query i,
    (i + 1) keys times (2 d_qk for q.k, 2 d_v for the weighted sum of v, plus
    the D weighting and the row sum), i.e. the causal half of QK^T and of P V."""
    pairs = T * (T + 1) // 2
    return B * H * pairs * (2 * dqk + 2 * dv + 2)


def time_events(fn, reps, stream):
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(reps):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / reps  # ms


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--chunk", type=int, default=64)
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--skip-step", action="store_true")
    ap.add_argument("--skip-extra", action="store_true")
    ap.add_argument("--skip-bwd", action="store_true")
    ap.add_argument("--skip-block", action="store_true")
    ap.add_argument("--skip-slstm", action="store_true")
    ap.add_argument("--skip-long", action="store_true")
    ap.add_argument("--skip-parallel", action="store_true")
    ap.add_argument("--profile-workload", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: every (batch, head) is independent, so the "
              "workload shards over GPUs without communication and the per-GPU rate is the "
              "one-GPU rate; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.profile_workload:
        profile_workload()
        return

    import torch

    import mlstm_matrix_memory_chunkwise_amd as M
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    M.load_library()

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    # ------------------------------------------------------------ chunkwise
    cfg = workloads.CONFIGS["d256_T8192"]
    log(f"bench: generating {cfg.describe()}")
    inp = workloads.make_chunkwise_inputs(cfg)
    d = {k: (None if v is None else v.to(dev)) for k, v in inp.items()}
    B, H, T, dqk, dv = cfg.B, cfg.H, cfg.T, cfg.dqk, cfg.dv
    h = torch.empty((B, H, T, dv), dtype=torch.bfloat16, device=dev)

    def chunk_pass(L):
        def run():
            M.mlstm_fwd_chunkwise(d["q"], d["k"], d["v"], d["i_pre"], d["f_pre"], d["o_pre"],
                                  d["C0"], d["n0"], d["m0"], chunk=L, out=h)
        return run

    run = chunk_pass(args.chunk)
    log(f"bench: warmup {args.warmup}")
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    # Clock settling: under a new sustained load the GPU's power management
    # first boosts, then overshoots into a slower phase for a few ms before it
    # settles (per-dispatch traces show ~0.5 ms, then up to ~0.75 ms, then
    # back).  Further untimed passes run until SETTLE_S seconds of this load
    # have elapsed, so that the timed steps see the sustained clock.
    settle_steps = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < SETTLE_S:
        for _ in range(10):
            run()
        torch.cuda.synchronize()
        settle_steps += 10
    log(f"bench: {settle_steps} settling passes")
    log(f"bench: timing {args.steps} steps")
    t0 = time.perf_counter()
    ms_events = time_events(run, args.steps, stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    flops, byts = chunk_algorithmic(B, H, T, dqk, dv, args.chunk, 4)
    sec = ms_events / 1e3
    tokens_per_s = B * T / sec
    result = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle_steps,
        "ms_per_step": wall_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"chunkwise mLSTM forward, bf16 q/k/v, fp32 gates/o-gate/state, "
                               f"B={B} H={H} T={T} d_qk={dqk} d_v={dv} chunk={args.chunk}, "
                               f"random initial state in, final state out",
                   "B": B, "H": H, "T": T, "d_qk": dqk, "d_v": dv, "chunk": args.chunk},
        "roofline": {
            "bound": "hbm",
            "achieved": byts / sec / 1e9,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": byts / sec / 1e9 / HBM_PEAK_GBS,
            "traffic": measured_traffic("chunkwise") if args.chunk == 64 else None,
        },
        "mfma": {"achieved_tflops": flops / sec / 1e12, "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                 "frac": flops / sec / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                 "algorithmic_gflop": flops / 1e9},
        "kernel_ms": ms_events,
        "algorithmic_bytes": byts,
    }

    if not args.skip_extra:
        other = 128 if args.chunk == 64 else 64
        run2 = chunk_pass(other)
        run2()
        torch.cuda.synchronize()
        ms2 = time_events(run2, max(3, args.steps // 2), stream)
        f2, b2 = chunk_algorithmic(B, H, T, dqk, dv, other, 4)
        result[f"chunk{other}"] = {"ms": ms2, "tokens_per_s": B * T / (ms2 / 1e3),
                                   "mfma_frac": f2 / (ms2 / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                                   "hbm_frac": b2 / (ms2 / 1e3) / 1e9 / HBM_PEAK_GBS,
                                   "algorithmic_bytes": b2,
                                   "traffic": measured_traffic("chunk128" if other == 128 else "chunkwise")}
        # no output gate (gating done at block level after GroupNorm)
        def run_noo():
            M.mlstm_fwd_chunkwise(d["q"], d["k"], d["v"], d["i_pre"], d["f_pre"], None,
                                  d["C0"], d["n0"], d["m0"], chunk=args.chunk, out=h)
        run_noo()
        torch.cuda.synchronize()
        ms3 = time_events(run_noo, max(3, args.steps // 2), stream)
        f3, b3 = chunk_algorithmic(B, H, T, dqk, dv, args.chunk, 0)
        result["no_ogate"] = {"ms": ms3, "tokens_per_s": B * T / (ms3 / 1e3),
                              "mfma_frac": f3 / (ms3 / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                              "hbm_frac": b3 / (ms3 / 1e3) / 1e9 / HBM_PEAK_GBS}
        # the block's gating done after the per-head normalization: the cell
        # without its gate, then group normalization + o-gate on its output,
        # against the cell with its own gate (what the normalization pass costs
        # on top of the cell)
        g7 = torch.Generator(device="cpu").manual_seed(cfg.seed + 7)
        gamma = (torch.randn((H, dv), generator=g7) * 0.5 + 1).to(dev)
        beta = (torch.randn((H, dv), generator=g7) * 0.5).to(dev)
        y = torch.empty_like(h)

        def run_pipe():
            M.mlstm_fwd_chunkwise(d["q"], d["k"], d["v"], d["i_pre"], d["f_pre"], None,
                                  d["C0"], d["n0"], d["m0"], chunk=args.chunk, out=h)
            M.mlstm_groupnorm_ogate(h, d["o_pre"], gamma, beta, 1e-5, out=y)

        run_pipe()
        torch.cuda.synchronize()
        ms_p = time_events(run_pipe, max(3, args.steps // 2), stream)
        result["cell_then_groupnorm"] = {
            "workload": "cell without o-gate, then per-head group normalization + o-gate (f32 "
                        "o~, affine) of its bf16 output, same inputs as the headline pass",
            "ms": ms_p, "tokens_per_s": B * T / (ms_p / 1e3),
            "cell_with_ogate_ms": ms_events,
            "extra_ms_over_cell_with_ogate": ms_p - ms_events,
            "extra_bytes": 2 * B * H * T * dv * 2,
        }
        del y, gamma, beta

    # ------------------------------------------------------------ backward
    if not args.skip_bwd:
        gen = torch.Generator(device="cpu").manual_seed(cfg.seed + 1)
        dh = torch.randn((B, H, T, dv), generator=gen).to(torch.bfloat16).to(dev)
        dC1 = torch.randn((B, H, dqk, dv), generator=gen).to(dev)
        dn1 = torch.randn((B, H, dqk), generator=gen).to(dev)
        run()   # h of these inputs
        torch.cuda.synchronize()
        bchunk = 64   # matrix products on bf16 MFMA (float32 accumulation)
        wsb = torch.empty(M.mlstm_bwd_chunkwise_workspace_bytes(
            M.Problem(B, H, T, dqk, dv, 1, 0, 0, 0), bchunk), dtype=torch.uint8, device=dev)

        def run_bwd():
            M.mlstm_bwd_chunkwise(d["q"], d["k"], d["v"], d["i_pre"], d["f_pre"], d["o_pre"],
                                  d["C0"], d["n0"], d["m0"], h, dh, dC1, dn1, chunk=bchunk,
                                  workspace=wsb)

        run_bwd()
        torch.cuda.synchronize()
        ms_b = time_events(run_bwd, max(3, args.steps // 4), stream)
        fb, bb = bwd_algorithmic(B, H, T, dqk, dv, bchunk, 4)
        result["backward"] = {
            "workload": f"chunkwise backward of the same pass (bf16 q/k/v/h/dh, f32 o-gate, state "
                        f"in, final-state gradient in), chunk {bchunk}; float32 gradients out",
            "ms": ms_b,
            "tokens_per_s": B * T / (ms_b / 1e3),
            "algorithmic_gflop": fb / 1e9,
            "algorithmic_bytes": bb,
            "hbm_frac": bb / (ms_b / 1e3) / 1e9 / HBM_PEAK_GBS,
            "mfma_frac": fb / (ms_b / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            # all five launches, from the counters (workspace states and
            # partial sums included)
            "traffic_bytes": measured_traffic("backward", "backward_calibrated_bytes_per_pass"),
            "workspace_bytes": wsb.numel(),
        }
        del dh, dC1, dn1, wsb
        torch.cuda.empty_cache()

    # ------------------------------------------------------------ block operations
    if not args.skip_block:
        gn, cv = block_inputs(dev)

        def run_gn():
            M.mlstm_groupnorm_ogate(gn["h"], gn["o"], gn["gamma"], gn["beta"], 1e-5, out=gn["y"])

        def run_conv():
            M.mlstm_causal_conv1d(cv["x"], cv["w"], cv["b"], cv["s"], out=cv["y"])

        for fn, key in ((run_gn, "groupnorm_ogate"), (run_conv, "causal_conv1d")):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            ms_x = time_events(fn, max(5, args.steps), stream)
            if key == "groupnorm_ogate":
                byts = groupnorm_algorithmic(**GN_SHAPE)
                wl = (f"per-head group normalization + o-gate of the cell output, h [{GN_SHAPE['B']},"
                      f"{GN_SHAPE['H']},{GN_SHAPE['T']},{GN_SHAPE['dv']}] bf16, f32 o-gate, affine")
                tr = measured_traffic("groupnorm")
            else:
                byts = conv_algorithmic(**CONV_SHAPE)
                wl = (f"causal depthwise conv1d K={CONV_SHAPE['K']}, x [{CONV_SHAPE['B']},"
                      f"{CONV_SHAPE['T']},{CONV_SHAPE['C']}] bf16, bias, carried window in and out")
                tr = measured_traffic("conv")
            gbs = byts / (ms_x / 1e3) / 1e9
            result[key] = {"workload": wl, "ms": ms_x,
                           "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS,
                                        "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                                        "traffic": tr},
                           "algorithmic_bytes": byts}
        del gn, cv
        torch.cuda.empty_cache()

    # ------------------------------------------------------------ sLSTM cell
    if not args.skip_slstm:
        import math
        B_, NH_, T_, DH_ = (SLSTM_SHAPE[k] for k in ("B", "NH", "T", "DH"))
        g = torch.Generator(device="cpu").manual_seed(11)
        wx = torch.randn((B_, NH_, T_, 4, DH_), generator=g)
        wx[:, :, :, 0] -= 1.0
        wx[:, :, :, 1] += 3.0
        wx = wx.to(torch.bfloat16).to(dev)
        Rm = (torch.randn((NH_, 4, DH_, DH_), generator=g) * (0.5 / math.sqrt(DH_))).to(dev)
        hs = torch.empty((B_, NH_, T_, DH_), dtype=torch.bfloat16, device=dev)

        def run_slstm():
            M.mlstm_slstm_fwd(wx, Rm, return_state=False, out=hs)

        run_slstm()
        torch.cuda.synchronize()
        ms_s = time_events(run_slstm, 3, stream)
        fl = slstm_flops(**SLSTM_SHAPE)
        tf = fl / (ms_s / 1e3) / 1e12
        result["slstm"] = {
            "workload": f"sLSTM forward, B={B_} NH={NH_} DH={DH_} T={T_}, bf16 wx and h, sigmoid "
                        f"forget gate, zero state; one workgroup per (batch, head)",
            "ms": ms_s, "tokens_per_s": B_ * T_ / (ms_s / 1e3), "us_per_step": ms_s * 1e3 / T_,
            "roofline": {"bound": "alu", "achieved": tf, "peak": FP32_VALU_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": tf / FP32_VALU_PEAK_TFLOPS, "traffic": None},
        }
        del wx, Rm, hs
        torch.cuda.empty_cache()

    # ------------------------------------------------------------ achievable rates
    # What this GPU reaches on plain library work, beside the datasheet peaks
    # the roofline fractions use: a 1 GiB device-to-device copy and a bf16
    # GEMM (torch.matmul on contiguous 2-D operands).
    if not args.skip_extra:
        xa = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        ya = torch.empty_like(xa)
        for _ in range(3):
            ya.copy_(xa)
        ms_c = time_events(lambda: ya.copy_(xa), 10, stream)
        copy_gbs = 2 * xa.numel() * 4 / (ms_c / 1e3) / 1e9
        del xa, ya
        ga = torch.randn((8192, 8192), device=dev).to(torch.bfloat16)
        gb = torch.randn((8192, 8192), device=dev).to(torch.bfloat16)
        gc = torch.empty((8192, 8192), dtype=torch.bfloat16, device=dev)
        for _ in range(5):   # library selection and first-call setup stay untimed
            torch.matmul(ga, gb, out=gc)
        torch.cuda.synchronize()
        ms_g = time_events(lambda: torch.matmul(ga, gb, out=gc), 10, stream)
        gemm_tf = 2 * 8192 ** 3 / (ms_g / 1e3) / 1e12
        del ga, gb, gc
        torch.cuda.empty_cache()
        result["achievable"] = {
            "copy_GBps": copy_gbs, "copy_frac_of_peak": copy_gbs / HBM_PEAK_GBS,
            "bf16_gemm_TFLOPs": gemm_tf, "gemm_frac_of_peak": gemm_tf / MFMA_BF16_PEAK_TFLOPS,
            "chunkwise_frac_of_copy": result["roofline"]["achieved"] / copy_gbs,
        }

    # ------------------------------------------------------------ CPU oracle
    if not args.skip_cpu:
        import oracle
        nheads = int(os.environ.get("MLSTM_BENCH_CPU_HEADS", "32"))
        sub = workloads.make_chunkwise_inputs(cfg, B=1, H=nheads)
        thr = oracle.max_threads()
        log(f"bench: oracle on {nheads} heads x {T} tokens, {thr} threads")
        t0 = time.perf_counter()
        oracle.recurrent(sub["q"], sub["k"], sub["v"], sub["i_pre"], sub["f_pre"], sub["o_pre"],
                         sub["C0"], sub["n0"], sub["m0"])
        cpu_s = time.perf_counter() - t0
        # tokens/s of the full workload = (token-heads/s) / H
        result["cpu_baseline"] = {
            "value": nheads * T / cpu_s / H,
            "unit": "tokens/s",
            "cores": min(thr, nheads),
            "kind": "oracle",
            "sample": f"{nheads} of the {B * H} heads (B=1, H={nheads}, T={T}, same distributions "
                      f"and seed recipe), fp64 sequential recurrence, {cpu_s:.2f} s wall; "
                      f"tokens/s scaled as token-heads/s / H={H}",
        }
    del d, inp, h
    torch.cuda.empty_cache()

    # ------------------------------------------------------------ decode step
    if not args.skip_step:
        cfg3 = workloads.CONFIGS["step_d512"]
        log(f"bench: generating {cfg3.describe()}")
        s = workloads.make_step_inputs(cfg3)
        ds = {k: (None if v is None else v.to(dev)) for k, v in s.items()}
        del s
        C, n, m = ds["C0"], ds["n0"], ds["m0"]
        hs = torch.empty((cfg3.B, cfg3.H, cfg3.dv), dtype=torch.bfloat16, device=dev)
        state = {"t": 0}

        def step():
            t = state["t"] % cfg3.T
            M.mlstm_step(ds["q"][t], ds["k"][t], ds["v"][t], ds["i_pre"][t], ds["f_pre"][t],
                         ds["o_pre"][t], C, n, m, inplace=True, out=hs)
            state["t"] += 1

        for _ in range(3):
            step()
        torch.cuda.synchronize()
        ms_step = time_events(step, cfg3.T, stream)
        sb = step_algorithmic(cfg3.B, cfg3.H, cfg3.dqk, cfg3.dv)
        gbs = sb / (ms_step / 1e3) / 1e9
        result["step"] = {
            "workload": f"decode step, bf16 q/k/v, fp32 state and o-gate, B={cfg3.B} H={cfg3.H} "
                        f"d_qk=d_v={cfg3.dqk}, {cfg3.T} consecutive in-place steps",
            "us_per_step": ms_step * 1e3,
            "tokens_per_s": cfg3.B / (ms_step / 1e3),
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": measured_traffic("step")},
            "algorithmic_bytes_per_step": sb,
        }
        del ds, C, n, m
        torch.cuda.empty_cache()

    # ------------------------------------------------------------ long context
    if not args.skip_long:
        cfg4 = workloads.CONFIGS["d256x512_T65536"]
        # the workload as given (16 heads: 128 workgroups, the sequence split
        # in 2), and with 4 heads (32 workgroups, split in 8)
        for key, heads in (("long_context", cfg4.H), ("long_context_4heads", 4)):
            log(f"bench: generating {cfg4.describe()} with H={heads}")
            d4 = {k: (None if v is None else v.to(dev))
                  for k, v in workloads.make_chunkwise_inputs(cfg4, H=heads).items()}
            B4, H4, T4, dqk4, dv4, L4 = cfg4.B, heads, cfg4.T, cfg4.dqk, cfg4.dv, cfg4.chunks[0]
            h4 = torch.empty((B4, H4, T4, dv4), dtype=torch.bfloat16, device=dev)

            def run_long():
                M.mlstm_fwd_chunkwise(d4["q"], d4["k"], d4["v"], d4["i_pre"], d4["f_pre"],
                                      d4["o_pre"], chunk=L4, out=h4)

            # warm-up, then untimed passes for SETTLE_S seconds (as for the
            # main line: the clock settles under a new sustained load)
            for _ in range(2):
                run_long()
            torch.cuda.synchronize()
            t_settle = time.perf_counter()
            while time.perf_counter() - t_settle < SETTLE_S:
                run_long()
                torch.cuda.synchronize()
            ms4 = time_events(run_long, 10, stream)
            f4, b4 = chunk_algorithmic(B4, H4, T4, dqk4, dv4, L4, 4, state_in=False)
            gbs4 = b4 / (ms4 / 1e3) / 1e9
            result[key] = {
                "workload": f"chunkwise forward, long context: bf16 q/k/v, fp32 gates/o-gate, B={B4} "
                            f"H={H4} T={T4} d_qk={dqk4} d_v={dv4} chunk={L4}, zero initial state, "
                            f"final state out",
                "ms": ms4, "tokens_per_s": B4 * T4 / (ms4 / 1e3),
                "roofline": {"bound": "hbm", "achieved": gbs4, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": gbs4 / HBM_PEAK_GBS,
                             # all launches of one call (states at the split points,
                             # forward, state copies)
                             "traffic": measured_traffic(key)},
                "mfma_frac": f4 / (ms4 / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                "algorithmic_bytes": b4, "algorithmic_gflop": f4 / 1e9,
            }
            del d4, h4
            torch.cuda.empty_cache()

    # ------------------------------------------------------------ parallel form
    if not args.skip_parallel:
        cfg1 = workloads.CONFIGS["d128_T2048"]
        log(f"bench: generating {cfg1.describe()}")
        d1 = {k: (None if v is None else v.to(dev))
              for k, v in workloads.make_chunkwise_inputs(cfg1).items()}
        B1, H1, T1, dqk1, dv1 = cfg1.B, cfg1.H, cfg1.T, cfg1.dqk, cfg1.dv
        h1 = torch.empty((B1, H1, T1, dv1), dtype=torch.bfloat16, device=dev)
        ws1 = torch.empty(M.mlstm_fwd_parallel_workspace_bytes(
            M.Problem(B1, H1, T1, dqk1, dv1, 1, 0, 0, 0)), dtype=torch.uint8, device=dev)

        def run_par():
            M.mlstm_fwd_parallel(d1["q"], d1["k"], d1["v"], d1["i_pre"], d1["f_pre"], d1["o_pre"],
                                 return_state=False, out=h1, workspace=ws1)

        for _ in range(3):
            run_par()
        torch.cuda.synchronize()
        ms1 = time_events(run_par, 20, stream)
        f1 = parallel_flops(B1, H1, T1, dqk1, dv1)
        tf1 = f1 / (ms1 / 1e3) / 1e12
        result["parallel_form"] = {
            "workload": f"parallel (quadratic) form, outputs only: bf16 q/k/v, fp32 gates/o-gate, "
                        f"B={B1} H={H1} T={T1} d_qk={dqk1} d_v={dv1}, zero initial state",
            "ms": ms1, "tokens_per_s": B1 * T1 / (ms1 / 1e3),
            "roofline": {"bound": "mfma", "achieved": tf1, "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": tf1 / MFMA_BF16_PEAK_TFLOPS, "traffic": None},
            "algorithmic_gflop": f1 / 1e9,
        }
        del d1, h1, ws1
        torch.cuda.empty_cache()

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
