"""Pins of the sLSTM oracle (``oracle/slstm.py``).

Checked against code it does not share: the unstabilized recurrence written
out unit by unit in plain Python (true-unit c and n, i = exp(i~), f = exp(f~)
or sigmoid(f~)), the closed form of the cell without recurrence (a weighted
mean of z), the constant-z invariant, the stabilizer-shift invariance,
split/resume and head independence.  Planted mistakes in a copy of the
oracle's source must fail a pin."""
from __future__ import annotations

import inspect
import math
import types

import numpy as np
import pytest

from oracle import slstm


def make_case(seed, B=2, NH=2, T=12, DH=3, scale_r=0.4, state=True):
    rng = np.random.default_rng(seed)
    wx = rng.normal(0, 1, (B, NH, T, 4, DH))
    wx[:, :, :, 0] = rng.normal(-0.5, 1.5, (B, NH, T, DH))    # i~
    wx[:, :, :, 1] = rng.normal(1.5, 1.0, (B, NH, T, DH))     # f~
    R = rng.normal(0, scale_r / math.sqrt(DH), (NH, 4, DH, DH))
    st = None
    if state:
        st = dict(c0=rng.normal(0, 1, (B, NH, DH)), n0=rng.uniform(0.5, 2.0, (B, NH, DH)),
                  m0=rng.normal(0, 1, (B, NH, DH)), h0=rng.normal(0, 0.5, (B, NH, DH)))
    return wx, R, st


def brute_force(wx, R, st, fgate):
    """True-unit recurrence, one unit at a time, plain Python floats."""
    B, NH, T, _, DH = wx.shape
    out = np.zeros((B, NH, T, DH))
    for b in range(B):
        for hd in range(NH):
            if st is None:
                c = [0.0] * DH
                n = [0.0] * DH
                h = [0.0] * DH
            else:
                c = [st["c0"][b, hd, u] * math.exp(st["m0"][b, hd, u]) for u in range(DH)]
                n = [st["n0"][b, hd, u] * math.exp(st["m0"][b, hd, u]) for u in range(DH)]
                h = [float(st["h0"][b, hd, u]) for u in range(DH)]
            for t in range(T):
                pre = [[float(wx[b, hd, t, g, u]) + sum(R[hd, g, u, v] * h[v] for v in range(DH))
                        for u in range(DH)] for g in range(4)]
                hn = []
                for u in range(DH):
                    i = math.exp(pre[0][u])
                    f = math.exp(pre[1][u]) if fgate == "exp" else 1.0 / (1.0 + math.exp(-pre[1][u]))
                    c[u] = f * c[u] + i * pre[2][u]
                    n[u] = f * n[u] + i
                    hn.append(1.0 / (1.0 + math.exp(-pre[3][u])) * c[u] / n[u])
                h = hn
                for u in range(DH):
                    out[b, hd, t, u] = h[u]
    return out


def check(mod):
    """All pins; returns the worst relative deviation."""
    worst = 0.0
    # 1. unstabilized brute force, both gates, with and without a state
    for seed, fgate, state in ((1, "sigmoid", True), (2, "exp", True), (3, "sigmoid", False)):
        wx, R, st = make_case(seed, state=state)
        if fgate == "exp":
            wx[:, :, :, 1] = np.random.default_rng(seed).normal(-0.1, 0.3, wx[:, :, :, 1].shape)
        kw = {} if st is None else st
        h, (c, n, m, hT) = mod.slstm_forward(wx, R, fgate=fgate, **kw)
        ref = brute_force(wx, R, st, fgate)
        worst = max(worst, np.max(np.abs(h - ref)) / np.max(np.abs(ref)))
    # 2. no recurrence, zero state: h_t = sigmoid(o~_t) * softmax-weighted mean of z_j (j <= t)
    wx, R, _ = make_case(4, T=15, state=False)
    R[:] = 0.0
    h, _ = mod.slstm_forward(wx, R, fgate="sigmoid")
    lf = np.minimum(wx[:, :, :, 1], 0) - np.log1p(np.exp(-np.abs(wx[:, :, :, 1])))
    F = np.cumsum(lf, axis=2)                                     # [B, NH, T, DH]
    for t in range(wx.shape[2]):
        logw = wx[:, :, :t + 1, 0] + F[:, :, t:t + 1] - F[:, :, :t + 1]   # i~_j + sum_{k=j+1..t} log f_k
        wgt = np.exp(logw - logw.max(axis=2, keepdims=True))
        mean = np.sum(wgt * wx[:, :, :t + 1, 2], axis=2) / np.sum(wgt, axis=2)
        ref = mean / (1.0 + np.exp(-wx[:, :, t, 3]))
        worst = max(worst, np.max(np.abs(h[:, :, t] - ref)))
    # 3. constant z (R_z = 0, z~ = zeta per unit, c0 = zeta n0): h = sigmoid(o~) zeta
    wx, R, st = make_case(5)
    zeta = np.random.default_rng(9).normal(0, 1, (wx.shape[0], wx.shape[1], wx.shape[4]))
    R[:, 2] = 0.0
    wx[:, :, :, 2] = zeta[:, :, None, :]
    st["c0"] = zeta * st["n0"]
    h, (_, _, _, _) = mod.slstm_forward(wx, R, **st)
    o = wx[:, :, :, 3] + 0.0
    # o~ includes R_o h_{t-1}: compare c/n through h / sigmoid(o~) with the oracle's own h chain
    hp = st["h0"]
    for t in range(wx.shape[2]):
        ot = o[:, :, t] + np.einsum("huv,bhv->bhu", R[:, 3], hp)
        ref = zeta / (1.0 + np.exp(-ot))
        worst = max(worst, np.max(np.abs(h[:, :, t] - ref)))
        hp = ref
    # 4. stabilizer shift: (c0 e^-s, n0 e^-s, m0 + s) leaves h unchanged
    wx, R, st = make_case(6)
    h1, _ = mod.slstm_forward(wx, R, **st)
    s = 3.25
    st2 = dict(st, c0=st["c0"] * math.exp(-s), n0=st["n0"] * math.exp(-s), m0=st["m0"] + s)
    h2, _ = mod.slstm_forward(wx, R, **st2)
    worst = max(worst, np.max(np.abs(h1 - h2)))
    # 5. head independence: another head's inputs do not reach head 0
    wx2 = wx.copy()
    wx2[:, 1] += 1.0
    h3, _ = mod.slstm_forward(wx2, R, **st)
    worst = max(worst, np.max(np.abs(h3[:, 0] - h1[:, 0])))
    return worst


def test_oracle_pins():
    assert check(slstm) < 1e-12


def test_split_resume_bitwise():
    wx, R, st = make_case(7, T=20)
    h, (c, n, m, hT) = slstm.slstm_forward(wx, R, **st)
    ha, (ca, na, ma, hA) = slstm.slstm_forward(wx[:, :, :9], R, **st)
    hb, (cb, nb, mb, hB) = slstm.slstm_forward(wx[:, :, 9:], R, c0=ca, n0=na, m0=ma, h0=hA)
    np.testing.assert_array_equal(np.concatenate([ha, hb], axis=2), h)
    for x, y in ((cb, c), (nb, n), (mb, m), (hB, hT)):
        np.testing.assert_array_equal(x, y)


MUTANTS = [
    ("z squashed by tanh", "c = fp * c + ip * z_t", "c = fp * c + ip * np.tanh(z_t)"),
    ("R transposed", '"hguv,bhv->bhgu"', '"hgvu,bhv->bhgu"'),
    ("stabilizer left out of the forget factor", "fp = np.exp(lf + m - m_new)", "fp = np.exp(lf)"),
    ("output gate not squashed", "hp = (1.0 / (1.0 + np.exp(-o_t))) * c / n", "hp = o_t * c / n"),
    ("normalizer without the input gate", "n = fp * n + ip", "n = fp * n + 1.0"),
]


@pytest.mark.parametrize("name,orig,mut", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutants_rejected(name, orig, mut):
    src = inspect.getsource(slstm)
    assert src.count(orig) == 1, name
    mod = types.ModuleType("slstm_mutant")
    exec(compile(src.replace(orig, mut), "slstm_mutant", "exec"), mod.__dict__)
    assert check(mod) > 1e-6, name
