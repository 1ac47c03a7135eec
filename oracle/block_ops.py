"""fp64 CPU oracle for the two block operations around the mLSTM cell.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this module; the HIP library
never calls it and shares no code with it.

Both follow the mLSTM block of the xLSTM post (llms.blog), section 4
"xLSTM Block Architecture and Residual Stacking", "mLSTM Block Structure"
(items 3 and 5 and the block figure; the sLSTM block of the same section
puts the same convolution before the sLSTM cell):

* ``groupnorm_ogate``: the cell output of each head is normalized over its
  d_v features (group normalization with one group per head, per token), then
  scaled by the output gate.  Reading: y = sigmoid(o~) * (gamma * (h - mean) /
  sqrt(var + eps) + beta), with the biased variance of the group, gamma and
  beta per (head, feature), and the o-gate applied after the normalization
  (the item names normalization first, then modulation by o_t).
* ``causal_conv1d``: a depthwise causal 1-D convolution with a small kernel
  (k = 4 on the page) over the token axis, channel by channel, on the paths
  that feed the cell.  Reading:
  y[t, c] = bias[c] + sum_{s<K} w[c, s] x[t - (K-1) + s, c], so w[c, K-1]
  multiplies the current token; inputs before the first token come from an
  optional carried window of the K-1 previous inputs (zeros when absent).
  The page names no activation after the convolution, so none is applied.

Arrays are converted to float64 first (exact for float32 and bfloat16).

Parity status: pinned (tests/test_oracle_block.py) against torch's own
group_norm and conv1d evaluated in float64 on the CPU (library routines),
closed forms (zero mean and unit variance of the normalized groups, the
impulse response of the convolution), invariances (shift and positive scale
of a group; the o-gate factorizes) and split/resume of the convolution, with
planted mistakes rejected.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):   # torch tensor (bfloat16 included)
        return x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def groupnorm_ogate(h, o_pre=None, gamma=None, beta=None, eps: float = 1e-5):
    """y[b, hd, t, :] = sigmoid(o~) * (gamma[hd] * (h - mean) / sqrt(var + eps) + beta[hd]).

    h, o_pre: [B, H, T, d_v]; gamma, beta: [H, d_v] (None: 1 and 0); the mean
    and the biased variance are over the d_v features of one (b, head, t).
    """
    x = _f64(h)
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    y = (x - mean) / np.sqrt(var + eps)
    if gamma is not None:
        y = y * _f64(gamma)[None, :, None, :]
    if beta is not None:
        y = y + _f64(beta)[None, :, None, :]
    if o_pre is not None:
        y = y * sigmoid(_f64(o_pre))
    return y


def causal_conv1d(x, w, bias=None, state=None):
    """Depthwise causal convolution over the token axis.

    x: [B, T, C]; w: [C, K]; bias: [C] or None; state: [B, K-1, C] (the K-1
    inputs before x[:, 0], oldest first) or None for zeros.
    Returns (y [B, T, C], new state [B, K-1, C]: the last K-1 inputs of the
    concatenation of state and x).
    """
    xs = _f64(x)
    wk = _f64(w)
    B, T, C = xs.shape
    K = wk.shape[1]
    prev = np.zeros((B, K - 1, C)) if state is None else _f64(state)
    full = np.concatenate([prev, xs], axis=1)          # token t sits at t + K - 1
    y = np.zeros((B, T, C))
    for t in range(T):
        for s in range(K):
            y[:, t, :] += wk[:, s][None, :] * full[:, t + s, :]
    if bias is not None:
        y += _f64(bias)[None, None, :]
    new_state = full[:, full.shape[1] - (K - 1):, :].copy() if K > 1 else np.zeros((B, 0, C))
    return y, new_state
