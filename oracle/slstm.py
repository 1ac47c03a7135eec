"""fp64 CPU oracle for the sLSTM forward cell (scalar memory, exponential
gating, normalizer and stabilizer, head-wise recurrent mixing).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this module; the HIP library
never calls it and shares no code with it.

Follows the xLSTM post (llms.blog), section 2 "sLSTM: Scalar Memory with
Exponential Gating and Normalization" (subsections "Exponential Gating",
"The Normalizer State and Numerical Stabilization", "Multi-Head Memory
Mixing").  Per time step t, head hd, unit u (all arithmetic in float64):

  pre_g   = wx[t, g, u] + sum_v R[hd, g, u, v] h_{t-1}[v]      g in (i, f, z, o)
  log f   = f~ (exponential forget gate) or log sigmoid(f~) (sigmoid gate)
  m_t     = max(log f + m_{t-1}, i~)
  c_t     = exp(log f + m_{t-1} - m_t) c_{t-1} + exp(i~ - m_t) z
  n_t     = exp(log f + m_{t-1} - m_t) n_{t-1} + exp(i~ - m_t)
  h_t     = sigmoid(o~) c_t / n_t

Readings where the page leaves a step open:
* wx holds the input projections W x_t + b of the four gates, already
  computed (the projections are generic GEMMs with trained weights), laid out
  [B, NH, T, 4, DH] with gate order (i, f, z, o).
* The recurrent matrices act within a head (block-diagonal over heads,
  R [NH, 4, DH, DH], pre = R h); one head over all units (NH = 1) is the
  dense form.  The page's sentence on mixing across heads is read as this
  head-structured R; NH = 1 covers a fully mixing R.
* z enters without a squashing nonlinearity, as the page states; the output
  gate is a sigmoid, as in the LSTM gates of section 1.
* The sigmoid forget gate enters the stabilizer through log sigmoid(f~), the
  exponential one through f~ itself (the page prints the latter).
* The state (c, n, m, h) is stored in the stabilized scale; zero initial
  state means c = n = h = 0 and m = 0.

Parity status: pinned (tests/test_oracle_slstm.py) against the unstabilized
recurrence written out unit by unit in plain Python (true-unit c and n with
exp gates), the closed form of the cell without recurrence (a weighted mean
of z), the constant-z invariant, the stabilizer-shift invariance,
split/resume, head independence, and planted mistakes.
"""
from __future__ import annotations

import numpy as np

FGATE_SIGMOID = "sigmoid"
FGATE_EXP = "exp"


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        return x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def log_sigmoid(x):
    return np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))


def slstm_forward(wx, R, c0=None, n0=None, m0=None, h0=None, fgate=FGATE_SIGMOID):
    """wx [B, NH, T, 4, DH], R [NH, 4, DH, DH]; state [B, NH, DH] each or None.

    Returns h [B, NH, T, DH] and the final state (c, n, m, h) [B, NH, DH].
    """
    x = _f64(wx)
    Rm = _f64(R)
    B, NH, T, four, DH = x.shape
    assert four == 4 and Rm.shape == (NH, 4, DH, DH)
    z0 = np.zeros((B, NH, DH))
    c = z0.copy() if c0 is None else _f64(c0).copy()
    n = z0.copy() if n0 is None else _f64(n0).copy()
    m = z0.copy() if m0 is None else _f64(m0).copy()
    hp = z0.copy() if h0 is None else _f64(h0).copy()
    out = np.zeros((B, NH, T, DH))
    for t in range(T):
        # recurrent contribution of each gate: R[hd, g] @ h_{t-1}[b, hd]
        rec = np.einsum("hguv,bhv->bhgu", Rm, hp)
        pre = x[:, :, t] + rec
        i_t, f_t, z_t, o_t = pre[:, :, 0], pre[:, :, 1], pre[:, :, 2], pre[:, :, 3]
        lf = f_t if fgate == FGATE_EXP else log_sigmoid(f_t)
        m_new = np.maximum(lf + m, i_t)
        fp = np.exp(lf + m - m_new)
        ip = np.exp(i_t - m_new)
        c = fp * c + ip * z_t
        n = fp * n + ip
        m = m_new
        hp = (1.0 / (1.0 + np.exp(-o_t))) * c / n
        out[:, :, t] = hp
    return out, (c, n, m, hp)
