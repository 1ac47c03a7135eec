"""Pins of the block-operation oracle (``oracle/block_ops.py``): the per-head
group normalization with output gate, and the causal depthwise convolution.

Each is checked against things it does not share code with: torch's own
CPU group_norm / conv1d in float64 (library routines), closed forms, invariances
and split/resume; planted mistakes in a copy of the oracle must fail a pin."""
from __future__ import annotations

import types

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import block_ops


def _gn_case(seed, B=2, H=3, T=5, dv=8):
    rng = np.random.default_rng(seed)
    return dict(h=rng.normal(0.3, 2.0, (B, H, T, dv)), o=rng.normal(0, 1, (B, H, T, dv)),
                gamma=rng.normal(1, 0.5, (H, dv)), beta=rng.normal(0, 0.5, (H, dv)))


def _gn_torch(c, eps):
    """torch.nn.functional.group_norm over channels (head, feature), one group
    per head, every (b, t) an independent sample; then the sigmoid o-gate."""
    h = torch.from_numpy(c["h"])
    B, H, T, dv = h.shape
    x = h.permute(0, 2, 1, 3).reshape(B * T, H * dv)
    y = F.group_norm(x, H, torch.from_numpy(c["gamma"]).reshape(-1),
                     torch.from_numpy(c["beta"]).reshape(-1), eps)
    y = y.reshape(B, T, H, dv).permute(0, 2, 1, 3)
    return (torch.sigmoid(torch.from_numpy(c["o"])) * y).numpy()


def check_gn(mod):
    """All pins of groupnorm_ogate; returns the worst deviation."""
    worst = 0.0
    for seed, eps in ((1, 1e-5), (2, 0.3)):
        c = _gn_case(seed)
        y = mod.groupnorm_ogate(c["h"], c["o"], c["gamma"], c["beta"], eps)
        worst = max(worst, np.max(np.abs(y - _gn_torch(c, eps))))
        # o factorizes: y(o) = sigmoid(o) * y(no o)
        y0 = mod.groupnorm_ogate(c["h"], None, c["gamma"], c["beta"], eps)
        worst = max(worst, np.max(np.abs(y - y0 / (1 + np.exp(-c["o"])))))
    # plain normalization: zero mean, variance var / (var + eps)
    c = _gn_case(3)
    eps = 0.25
    y = mod.groupnorm_ogate(c["h"], eps=eps)
    var = c["h"].var(axis=-1)
    worst = max(worst, np.max(np.abs(y.mean(axis=-1))))
    worst = max(worst, np.max(np.abs(y.var(axis=-1) - var / (var + eps))))
    # shift and positive scale of a group leave it unchanged (eps = 0)
    a = 3.7
    y1 = mod.groupnorm_ogate(c["h"], c["o"], c["gamma"], c["beta"], 0.0)
    y2 = mod.groupnorm_ogate(a * c["h"] - 1.25, c["o"], c["gamma"], c["beta"], 0.0)
    worst = max(worst, np.max(np.abs(y1 - y2)))
    # one group by hand: features (1, 2, 3, 6): mean 3, var 3.5
    h = np.array([1.0, 2.0, 3.0, 6.0]).reshape(1, 1, 1, 4)
    ref = (np.array([1.0, 2.0, 3.0, 6.0]) - 3.0) / np.sqrt(3.5 + 0.5)
    worst = max(worst, np.max(np.abs(mod.groupnorm_ogate(h, eps=0.5).reshape(-1) - ref)))
    return worst


def test_groupnorm_pins():
    assert check_gn(block_ops) < 1e-12


def _conv_case(seed, B=2, T=11, C=5, K=4):
    rng = np.random.default_rng(seed)
    return dict(x=rng.normal(0, 1, (B, T, C)), w=rng.normal(0, 1, (C, K)), b=rng.normal(0, 1, C),
                s=rng.normal(0, 1, (B, K - 1, C)))


def _conv_torch(x, w, b):
    """torch conv1d, depthwise (groups = C), left padding K-1: the causal form."""
    xt = torch.from_numpy(x).permute(0, 2, 1)                     # [B, C, T]
    C, K = w.shape
    y = F.conv1d(F.pad(xt, (K - 1, 0)), torch.from_numpy(w).reshape(C, 1, K),
                 torch.from_numpy(b), groups=C)
    return y.permute(0, 2, 1).numpy()


def _mx(a):
    return float(np.max(np.abs(a))) if np.size(a) else 0.0


def check_conv(mod):
    worst = 0.0
    for seed, K in ((1, 4), (2, 1), (3, 3), (4, 8)):
        c = _conv_case(seed, K=K)
        y, st = mod.causal_conv1d(c["x"], c["w"], c["b"])
        worst = max(worst, np.max(np.abs(y - _conv_torch(c["x"], c["w"], c["b"]))))
        if K > 1:   # the carried window is the last K-1 inputs
            worst = max(worst, np.max(np.abs(st - c["x"][:, -(K - 1):, :])))
        # split / resume: two halves with the carried window == one pass
        for cut in (1, 5):
            ya, sa = mod.causal_conv1d(c["x"][:, :cut], c["w"], c["b"], c["s"][:, :K - 1])
            yb, sb = mod.causal_conv1d(c["x"][:, cut:], c["w"], c["b"], sa)
            yf, sf = mod.causal_conv1d(c["x"], c["w"], c["b"], c["s"][:, :K - 1])
            worst = max(worst, _mx(np.concatenate([ya, yb], 1) - yf), _mx(sb - sf))
    # the carried window equals the inputs it stands for
    c = _conv_case(5)
    full = np.concatenate([c["s"], c["x"]], axis=1)
    y_full = _conv_torch(full, c["w"], c["b"])[:, 3:]
    y, _ = mod.causal_conv1d(c["x"], c["w"], c["b"], c["s"])
    worst = max(worst, np.max(np.abs(y - y_full)))
    # impulse response: a unit input at t0 in channel c gives w[c, K-1-s] at t0 + s
    T, C, K = 9, 3, 4
    x = np.zeros((1, T, C))
    x[0, 2, 1] = 1.0
    w = np.arange(1.0, 1.0 + C * K).reshape(C, K)
    y, _ = mod.causal_conv1d(x, w)
    ref = np.zeros((1, T, C))
    for s in range(K):
        ref[0, 2 + s, 1] = w[1, K - 1 - s]
    worst = max(worst, np.max(np.abs(y - ref)))
    return worst


def test_conv_pins():
    assert check_conv(block_ops) < 1e-12


def _mutant(gn=None, conv=None):
    """A copy of the oracle module with one function replaced."""
    m = types.SimpleNamespace(groupnorm_ogate=block_ops.groupnorm_ogate,
                              causal_conv1d=block_ops.causal_conv1d)
    if gn is not None:
        m.groupnorm_ogate = gn
    if conv is not None:
        m.causal_conv1d = conv
    return m


def _gn_unbiased(h, o_pre=None, gamma=None, beta=None, eps=1e-5):
    x = np.asarray(h, dtype=np.float64)
    y = (x - x.mean(-1, keepdims=True)) / np.sqrt(x.var(-1, ddof=1, keepdims=True) + eps)
    y = y * (1 if gamma is None else np.asarray(gamma)[None, :, None, :])
    y = y + (0 if beta is None else np.asarray(beta)[None, :, None, :])
    return y * (1 if o_pre is None else block_ops.sigmoid(np.asarray(o_pre)))


def _gn_gate_before(h, o_pre=None, gamma=None, beta=None, eps=1e-5):
    x = np.asarray(h, dtype=np.float64)
    if o_pre is not None:
        x = x * block_ops.sigmoid(np.asarray(o_pre))
    return block_ops.groupnorm_ogate(x, None, gamma, beta, eps)


def _conv_flipped(x, w, bias=None, state=None):
    return block_ops.causal_conv1d(x, np.asarray(w)[:, ::-1], bias, state)


def _conv_no_state(x, w, bias=None, state=None):
    return block_ops.causal_conv1d(x, w, bias, None)


MUTANTS = [
    ("unbiased variance", dict(gn=_gn_unbiased)),
    ("o-gate before the normalization", dict(gn=_gn_gate_before)),
    ("kernel taps reversed", dict(conv=_conv_flipped)),
    ("carried window ignored", dict(conv=_conv_no_state)),
]


@pytest.mark.parametrize("name,kw", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_block_mutants_rejected(name, kw):
    m = _mutant(**kw)
    assert max(check_gn(m), check_conv(m)) > 1e-6, name
