"""Seeded synthetic inputs for the mLSTM cell forward pass.

This module holds only input recipes: shapes, dtypes, distributions and seeds.
It computes nothing of the method itself.  Both the HIP path's callers (tests,
benchmark, smoke check) and the oracle's callers draw their inputs here, so the
two sides always see the same bits.

The pages train on language-model data and print no layer shapes, so the
workloads are synthetic tensors shaped like language-model mLSTM layers:

  tiny_fp32        fp32, B=1, H=1, T=64, d_qk=d_v=16, chunk 16; zero state
  d128_T2048       bf16 q/k/v, fp32 gates and state, B=4, H=4, T=2048,
                   d=128, chunk 64
  d256_T8192       bf16, B=8, H=8, T=8192, d=256, chunk 64 and 128;
                   i~ ~ N(-2,3), f~ ~ N(4,2); random initial state N(0,1)
  step_d512        decode step, bf16 q/k/v, fp32 state, B=128, H=8, d=512,
                   256 steps; initial state N(0,1); per-step gates as
                   tiny_fp32
  d256x512_T65536  bf16, B=1, H=16, T=65536, d_qk=256, d_v=512, chunk 128;
                   f~ ~ N(6,1), i~ ~ N(0,2); zero initial state

The seed index of each (0 to 4, in the order above) fixes its generator.

Recipe (every config): a CPU ``torch.Generator`` seeded with 1000 + index.
Draw order: q, k, v, i~, f~, o~, then (if the state is random) C0, n0, m0.
Every draw is float32 ``normal(mean, std)`` (std is the second number).
k is multiplied by 1/sqrt(d_qk) in float32 before any cast.  For bf16 configs
q, k, v are then rounded to bfloat16 (round to nearest even); gates, o~ and the
state stay float32.  The forget gate goes through logsigmoid (sigmoid gate).
For step_d512 the state is drawn first, then per step s = 0..S-1 the tuple
(q, k, v, i~, f~, o~), each as one [S,B,H,...] tensor in that order.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple

import torch


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    index: int
    dtype: str            # "f32" or "bf16": dtype of q, k, v and h
    B: int
    H: int
    T: int                # tokens (for the step config: number of steps)
    dqk: int
    dv: int
    chunks: Tuple[int, ...]
    i_dist: Tuple[float, float]
    f_dist: Tuple[float, float]
    o_dist: Optional[Tuple[float, float]]   # None: no output gate (o = 1)
    random_state: bool
    fgate: str = "sigmoid"
    kind: str = "chunkwise"                  # "chunkwise" or "step"

    @property
    def seed(self) -> int:
        return 1000 + self.index

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def describe(self) -> str:
        return (f"{self.name}: {self.kind} {self.dtype} B={self.B} H={self.H} "
                f"T={self.T} d_qk={self.dqk} d_v={self.dv} chunk={self.chunks}")


CONFIGS: Dict[str, Config] = {
    "tiny_fp32": Config("tiny_fp32", 0, "f32", 1, 1, 64, 16, 16, (16,), (0.0, 1.0), (3.0, 1.0),
                 (0.0, 1.0), False),
    "d128_T2048": Config("d128_T2048", 1, "bf16", 4, 4, 2048, 128, 128, (64,), (0.0, 1.0), (3.0, 1.0),
                 (0.0, 1.0), False),
    "d256_T8192": Config("d256_T8192", 2, "bf16", 8, 8, 8192, 256, 256, (64, 128), (-2.0, 3.0),
                 (4.0, 2.0), (0.0, 1.0), True),
    "step_d512": Config("step_d512", 3, "bf16", 128, 8, 256, 512, 512, (), (0.0, 1.0), (3.0, 1.0),
                 (0.0, 1.0), True, kind="step"),
    "d256x512_T65536": Config("d256x512_T65536", 4, "bf16", 1, 16, 65536, 256, 512, (128,), (0.0, 2.0),
                 (6.0, 1.0), (0.0, 1.0), False),
}


def _normal(gen: torch.Generator, shape, mean: float, std: float) -> torch.Tensor:
    out = torch.empty(shape, dtype=torch.float32)
    out.normal_(mean, std, generator=gen)
    return out


def make_chunkwise_inputs(cfg: Config, *, B: Optional[int] = None,
                          H: Optional[int] = None, T: Optional[int] = None,
                          with_o: bool = True, seed: Optional[int] = None
                          ) -> Dict[str, Optional[torch.Tensor]]:
    """Inputs for a whole-sequence call, on the CPU.

    B, H, T override the config's sizes (for reduced parity cases that keep the
    config's distributions).  Returns a dict with q, k, v (cfg dtype), i_pre,
    f_pre (float32 [B,H,T]), o_pre (float32 [B,H,T,dv] or None) and C0, n0, m0
    (float32, or None for the zero state).
    """
    B = cfg.B if B is None else B
    H = cfg.H if H is None else H
    T = cfg.T if T is None else T
    gen = torch.Generator(device="cpu")
    gen.manual_seed(cfg.seed if seed is None else seed)
    q = _normal(gen, (B, H, T, cfg.dqk), 0.0, 1.0)
    k = _normal(gen, (B, H, T, cfg.dqk), 0.0, 1.0) * (1.0 / math.sqrt(cfg.dqk))
    v = _normal(gen, (B, H, T, cfg.dv), 0.0, 1.0)
    i_pre = _normal(gen, (B, H, T), *cfg.i_dist)
    f_pre = _normal(gen, (B, H, T), *cfg.f_dist)
    o_pre = _normal(gen, (B, H, T, cfg.dv), *cfg.o_dist) if (with_o and cfg.o_dist) else None
    C0 = n0 = m0 = None
    if cfg.random_state:
        C0 = _normal(gen, (B, H, cfg.dqk, cfg.dv), 0.0, 1.0)
        n0 = _normal(gen, (B, H, cfg.dqk), 0.0, 1.0)
        m0 = _normal(gen, (B, H), 0.0, 1.0)
    dt = cfg.torch_dtype
    return dict(q=q.to(dt), k=k.to(dt), v=v.to(dt), i_pre=i_pre, f_pre=f_pre,
                o_pre=o_pre, C0=C0, n0=n0, m0=m0)


def make_step_inputs(cfg: Config, *, B: Optional[int] = None,
                     H: Optional[int] = None, steps: Optional[int] = None,
                     with_o: bool = True, seed: Optional[int] = None
                     ) -> Dict[str, Optional[torch.Tensor]]:
    """Inputs for a run of consecutive decode steps, on the CPU.

    Returns C0 [B,H,dqk,dv], n0 [B,H,dqk], m0 [B,H] (float32) and per-step
    q, k [S,B,H,dqk], v [S,B,H,dv] (cfg dtype), i_pre, f_pre [S,B,H] and
    o_pre [S,B,H,dv] (float32, or None).
    """
    B = cfg.B if B is None else B
    H = cfg.H if H is None else H
    S = cfg.T if steps is None else steps
    gen = torch.Generator(device="cpu")
    gen.manual_seed(cfg.seed if seed is None else seed)
    C0 = _normal(gen, (B, H, cfg.dqk, cfg.dv), 0.0, 1.0)
    n0 = _normal(gen, (B, H, cfg.dqk), 0.0, 1.0)
    m0 = _normal(gen, (B, H), 0.0, 1.0)
    q = _normal(gen, (S, B, H, cfg.dqk), 0.0, 1.0)
    k = _normal(gen, (S, B, H, cfg.dqk), 0.0, 1.0) * (1.0 / math.sqrt(cfg.dqk))
    v = _normal(gen, (S, B, H, cfg.dv), 0.0, 1.0)
    i_pre = _normal(gen, (S, B, H), *cfg.i_dist)
    f_pre = _normal(gen, (S, B, H), *cfg.f_dist)
    o_pre = _normal(gen, (S, B, H, cfg.dv), *cfg.o_dist) if (with_o and cfg.o_dist) else None
    dt = cfg.torch_dtype
    return dict(q=q.to(dt), k=k.to(dt), v=v.to(dt), i_pre=i_pre, f_pre=f_pre,
                o_pre=o_pre, C0=C0, n0=n0, m0=m0)


def make_large_device_inputs(B: int, H: int, T: int, dqk: int, dv: int, seed: int,
                             device) -> Dict[str, Optional[torch.Tensor]]:
    """Inputs of a whole-sequence problem too large to draw on the host, drawn
    on `device` with a device generator seeded with `seed`.  Same recipe as the
    workloads above otherwise (draw order q, k, v, i~, f~; float32 normal draws;
    k scaled by 1/sqrt(d_qk) before the cast; q, k, v rounded to bfloat16):
    q, k, v ~ N(0,1), i~ ~ N(-1, 2), f~ ~ N(3, 1); no output gate and a zero
    initial state.  A check on the host copies slices of these same tensors."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def draw(shape, mean, std, scale=1.0, bf16=False):
        x = torch.empty(shape, dtype=torch.float32, device=device)
        x.normal_(mean, std, generator=g)
        if scale != 1.0:
            x.mul_(scale)
        return x.to(torch.bfloat16) if bf16 else x

    q = draw((B, H, T, dqk), 0.0, 1.0, bf16=True)
    k = draw((B, H, T, dqk), 0.0, 1.0, scale=1.0 / math.sqrt(dqk), bf16=True)
    v = draw((B, H, T, dv), 0.0, 1.0, bf16=True)
    i_pre = draw((B, H, T), -1.0, 2.0)
    f_pre = draw((B, H, T), 3.0, 1.0)
    return dict(q=q, k=k, v=v, i_pre=i_pre, f_pre=f_pre, o_pre=None, C0=None, n0=None, m0=None)


def make_large_device_step(B: int, H: int, dqk: int, dv: int, seed: int,
                           device) -> Dict[str, torch.Tensor]:
    """One decode step over a state too large to draw on the host: state C~,
    n~, m ~ N(0,1) drawn first, then q, k, v (bf16, k scaled by 1/sqrt(d_qk)),
    i~ ~ N(0,1), f~ ~ N(3,1), o~ ~ N(0,1), on `device` with a generator seeded
    with `seed`."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def draw(shape, mean, std):
        x = torch.empty(shape, dtype=torch.float32, device=device)
        x.normal_(mean, std, generator=g)
        return x

    C = draw((B, H, dqk, dv), 0.0, 1.0)
    n = draw((B, H, dqk), 0.0, 1.0)
    m = draw((B, H), 0.0, 1.0)
    q = draw((B, H, dqk), 0.0, 1.0).to(torch.bfloat16)
    k = (draw((B, H, dqk), 0.0, 1.0) / math.sqrt(dqk)).to(torch.bfloat16)
    v = draw((B, H, dv), 0.0, 1.0).to(torch.bfloat16)
    i_pre = draw((B, H), 0.0, 1.0)
    f_pre = draw((B, H), 3.0, 1.0)
    o_pre = draw((B, H, dv), 0.0, 1.0)
    return dict(q=q, k=k, v=v, i_pre=i_pre, f_pre=f_pre, o_pre=o_pre, C=C, n=n, m=m)


def make_large_device_block_inputs(seed: int, device) -> Dict[str, torch.Tensor]:
    """Block-operation inputs past 2^31 elements, drawn on `device` with a
    generator seeded with `seed`, in this order: group normalization h
    [1, 1100, 8192, 256] bf16 ~ N(0,1), o~ float32 ~ N(0,1), gamma ~ N(1, 0.5)
    and beta ~ N(0, 0.5) [1100, 256]; causal conv x [8, 131200, 2048] bf16
    ~ N(0,1), w [2048, 4] ~ N(0, 1/2), bias [2048] ~ N(0,1)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def draw(shape, mean, std, bf16=False):
        x = torch.empty(shape, dtype=torch.float32, device=device)
        x.normal_(mean, std, generator=g)
        return x.to(torch.bfloat16) if bf16 else x

    out = dict(h=draw((1, 1100, 8192, 256), 0.0, 1.0, bf16=True))
    out["o_pre"] = draw((1, 1100, 8192, 256), 0.0, 1.0)
    out["gamma"] = draw((1100, 256), 1.0, 0.5)
    out["beta"] = draw((1100, 256), 0.0, 0.5)
    out["x"] = draw((8, 131200, 2048), 0.0, 1.0, bf16=True)
    out["w"] = draw((2048, 4), 0.0, 0.5)
    out["bias"] = draw((2048,), 0.0, 1.0)
    return out


def make_large_device_grads(B: int, H: int, T: int, dqk: int, dv: int, seed: int,
                            device) -> Dict[str, torch.Tensor]:
    """Output gradients for the backward of a problem from
    make_large_device_inputs, drawn on `device` with a generator seeded with
    `seed`: dh [B,H,T,d_v] bf16 ~ N(0,1), then dC1 [B,H,d_qk,d_v] and dn1
    [B,H,d_qk] float32 ~ N(0,1)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def draw(shape):
        x = torch.empty(shape, dtype=torch.float32, device=device)
        x.normal_(0.0, 1.0, generator=g)
        return x

    return dict(dh=draw((B, H, T, dv)).to(torch.bfloat16), dC1=draw((B, H, dqk, dv)),
                dn1=draw((B, H, dqk)))


def make_large_device_slstm(B: int, NH: int, T: int, DH: int, seed: int,
                            device) -> Dict[str, torch.Tensor]:
    """sLSTM inputs past 2^31 elements, drawn on `device` with a generator
    seeded with `seed`: wx [B,NH,T,4,DH] float32 ~ N(0,1) with the input gate
    row ~ N(-1, 1) and the forget gate row ~ N(3, 1), rounded to bfloat16;
    then R [NH,4,DH,DH] float32 ~ N(0, 0.5/sqrt(DH)); zero initial state."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    wx = torch.empty((B, NH, T, 4, DH), dtype=torch.float32, device=device)
    wx.normal_(0.0, 1.0, generator=g)
    wx[:, :, :, 0].add_(-1.0)
    wx[:, :, :, 1].add_(3.0)
    wx = wx.to(torch.bfloat16)
    R = torch.empty((NH, 4, DH, DH), dtype=torch.float32, device=device)
    R.normal_(0.0, 0.5 / math.sqrt(DH), generator=g)
    return dict(wx=wx, R=R)
