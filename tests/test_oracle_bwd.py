"""Pins of the gradient oracle (``oracle/mlstm_oracle_bwd.c``).

The gradient oracle differentiates the token recurrence by hand in reverse
mode.  It is pinned against things it does not share code with:

* central finite differences of the *forward* oracle (itself pinned by the
  forward tests), for every input, on small cases that cross a recompute
  segment boundary, for both forget gates, with and without the o-gate, the
  initial state and the final-state gradient;
* the closed form of a single token from the zero state (both branches of
  the denominator);
* the closed form of causal linear attention (f = 1, i = 1, |n.q| < 1:
  h_t = sum_{j<=t} (q_t.k_j) v_j), whose gradients are plain matrix products;
* planted mistakes in a copy of the gradient source, each rejected by the
  finite-difference pin.

The loss is L = sum dh . h + e^{m_T - m_T*} (<dC1, C~_T> + <dn1, n~_T>) with
m_T* the unperturbed final maximum, i.e. dC1, dn1 are gradients of the final
memory in the scale of the stored final state.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle


def make_case(seed, B=1, H=2, T=70, dqk=4, dv=3, fgate="sigmoid", o=True, state=True, dstate=True):
    rng = np.random.default_rng(seed)
    c = dict(
        q=rng.normal(0, 1, (B, H, T, dqk)),
        k=rng.normal(0, 1, (B, H, T, dqk)) / np.sqrt(dqk),
        v=rng.normal(0, 1, (B, H, T, dv)),
        i_pre=rng.normal(-0.5, 1.0, (B, H, T)),
        f_pre=rng.normal(2.0, 1.0, (B, H, T)) if fgate == "sigmoid" else rng.normal(-0.2, 0.3, (B, H, T)),
        o_pre=rng.normal(0, 1, (B, H, T, dv)) if o else None,
        C0=rng.normal(0, 1, (B, H, dqk, dv)) if state else None,
        n0=rng.normal(0, 1, (B, H, dqk)) if state else None,
        m0=rng.normal(0, 1, (B, H)) if state else None,
        dh=rng.normal(0, 1, (B, H, T, dv)),
        dC1=rng.normal(0, 1, (B, H, dqk, dv)) if dstate else None,
        dn1=rng.normal(0, 1, (B, H, dqk)) if dstate else None,
    )
    return c


def loss(c, fgate, m_ref=None, lib=None):
    h, C1, n1, m1 = oracle.recurrent(c["q"], c["k"], c["v"], c["i_pre"], c["f_pre"], c["o_pre"],
                                     c["C0"], c["n0"], c["m0"], fgate=fgate, lib=lib)
    L = float(np.sum(c["dh"] * h))
    if c["dC1"] is not None:
        ref = m1 if m_ref is None else m_ref
        s = np.exp(m1 - ref)[..., None]
        L += float(np.sum(s[..., None] * c["dC1"] * C1) + np.sum(s * c["dn1"] * n1))
    return L, m1


GRAD_OF = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("i_pre", "di"), ("f_pre", "df"),
           ("o_pre", "do"), ("C0", "dC0"), ("n0", "dn0"), ("m0", "dm0")]


def fd_check(c, fgate, g, eps=1e-6, n_per=6, seed=0, lib=None):
    """Largest |analytic - central difference| / (1 + |central difference|)
    over a sample of entries of every input."""
    _, m_ref = loss(c, fgate, lib=lib)
    rng = np.random.default_rng(seed)
    worst = 0.0
    for name, gname in GRAD_OF:
        if c[name] is None:
            continue
        x = c[name]
        flat = x.reshape(-1)
        idx = rng.choice(flat.size, size=min(n_per, flat.size), replace=False)
        for j in idx:
            keep = flat[j]
            flat[j] = keep + eps
            lp, _ = loss(c, fgate, m_ref, lib=lib)
            flat[j] = keep - eps
            lm, _ = loss(c, fgate, m_ref, lib=lib)
            flat[j] = keep
            fd = (lp - lm) / (2 * eps)
            an = g[gname].reshape(-1)[j]
            worst = max(worst, abs(an - fd) / (1.0 + abs(fd)))
    return worst


def grads(c, fgate, lib=None):
    return oracle.backward(c["q"], c["k"], c["v"], c["i_pre"], c["f_pre"], c["o_pre"],
                           c["C0"], c["n0"], c["m0"], c["dh"], c["dC1"], c["dn1"],
                           fgate=fgate, lib=lib)


FD_CASES = [
    (1, "sigmoid", True, True, True),
    (2, "exp", True, True, True),
    (3, "sigmoid", False, False, False),
    (4, "sigmoid", True, False, True),
    (5, "exp", False, True, False),
]


@pytest.mark.parametrize("seed,fgate,o,state,dstate", FD_CASES)
def test_finite_differences(seed, fgate, o, state, dstate):
    """Every gradient against central differences of the forward oracle
    (T = 70 crosses the 64-token recompute segment)."""
    c = make_case(seed, fgate=fgate, o=o, state=state, dstate=dstate)
    g = grads(c, fgate)
    assert fd_check(c, fgate, g, seed=seed) < 1e-6


def test_single_token_closed_form():
    """One token from the zero state, no o-gate: h = i (q.k) v / max(|i q.k|, 1)."""
    rng = np.random.default_rng(11)
    for big in (False, True):
        dqk, dv = 5, 3
        q = rng.normal(0, 1, dqk)
        k = rng.normal(0, 1, dqk) / np.sqrt(dqk)
        v = rng.normal(0, 1, dv)
        dh = rng.normal(0, 1, dv)
        qk = q @ k
        ip = np.log(4.0 / abs(qk)) if big else np.log(0.25 / abs(qk))   # |i q.k| = 4 or 1/4
        i = np.exp(ip)
        e = lambda a: np.asarray(a, dtype=np.float64).reshape((1, 1, 1) + np.shape(a))  # noqa: E731
        g = oracle.backward(e(q), e(k), e(v), e(ip), e(1.0), None, None, None, None, e(dh))
        if big:   # h = sign(q.k) v
            ref = dict(dq=0 * q, dk=0 * k, dv=np.sign(qk) * dh, di=0.0)
        else:     # h = i (q.k) v
            ref = dict(dq=i * (dh @ v) * k, dk=i * (dh @ v) * q, dv=i * qk * dh, di=i * qk * (dh @ v))
        for name, val in ref.items():
            np.testing.assert_allclose(g[name].reshape(np.shape(val)), val, rtol=1e-12, atol=1e-14)
        assert abs(g["df"].item()) < 1e-15   # f multiplies the zero initial state


def test_linear_attention_closed_form():
    """f = 1, i = 1 and |n.q| < 1 everywhere: the cell is causal linear
    attention h = tril(Q K^T) V, with dQ = tril(dH V^T) K, dK = tril(dH V^T)^T Q,
    dV = tril(Q K^T)^T dH."""
    rng = np.random.default_rng(5)
    T, dqk, dv = 40, 6, 4
    q = rng.normal(0, 1, (T, dqk)) * 0.1
    k = rng.normal(0, 1, (T, dqk)) * 0.1 / np.sqrt(dqk)
    v = rng.normal(0, 1, (T, dv))
    dh = rng.normal(0, 1, (T, dv))
    S = np.tril(q @ k.T)
    n = np.cumsum(k, axis=0)
    assert np.max(np.abs(np.sum(n * q, axis=1))) < 1.0
    e = lambda a: np.asarray(a, dtype=np.float64)[None, None]  # noqa: E731
    g = oracle.backward(e(q), e(k), e(v), e(np.zeros(T)), e(np.zeros(T)), None, None, None, None,
                        e(dh), fgate="exp")
    Gm = np.tril(dh @ v.T)
    np.testing.assert_allclose(g["dq"][0, 0], Gm @ k, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(g["dk"][0, 0], Gm.T @ q, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(g["dv"][0, 0], S.T @ dh, rtol=1e-11, atol=1e-13)
    # d i~_j = k_j . dk_j (i = exp(i~) = 1 here); d f~ via the log-forget identity
    np.testing.assert_allclose(g["di"][0, 0], np.sum(k * (Gm.T @ q), axis=1), rtol=1e-11, atol=1e-13)


BWD_MUTANTS = [
    ("denominator term dropped from the gradient",
     "Gn[a] += dnq * qt[a];", "Gn[a] += 0.0 * dnq * qt[a];"),
    ("forget-gate derivative without f (1 - f)",
     "? f * (1.0 - f) : f", "? f : f"),
    ("memory gradient not decayed",
     "for (int64_t x = 0; x < S; ++x) G[x] *= f;", "for (int64_t x = 0; x < S; ++x) G[x] *= 1.0;"),
    ("key gradient without the normalizer path",
     "dk[tok * dqk + a] = i * (gv + Gn[a]);", "dk[tok * dqk + a] = i * gv;"),
    ("forget gradient against the updated state",
     "fc += GC[a * dv + b] * Cp[a * dv + b];", "fc += GC[a * dv + b] * Ct[a * dv + b];"),
]


@pytest.mark.parametrize("name,orig,mut", BWD_MUTANTS, ids=[m[0] for m in BWD_MUTANTS])
def test_mutants_rejected(tmp_path, name, orig, mut):
    src = oracle.bwd_source_text()
    assert src.count(orig) == 1, name
    lib = oracle.load_library(oracle.build_variant(oracle.source_text(), str(tmp_path / "libmut.so"),
                                                   bwd_text=src.replace(orig, mut)))
    worst = 0.0
    for seed, fgate, o, state, dstate in FD_CASES[:3]:
        c = make_case(seed, T=20, fgate=fgate, o=o, state=state, dstate=dstate)
        worst = max(worst, fd_check(c, fgate, grads(c, fgate, lib=lib), seed=seed))
    assert worst > 1e-4, name


def test_empty_sequence_closed_form():
    """T = 0: the final memory is the initial one, so its gradient passes
    through (dC0 = dC1, dn0 = dn1 in the stored scale) and the derivative
    through e^{m0} is <dC1, C~0> + <dn1, n~0>; the forward returns the state."""
    import numpy as np
    import torch
    import oracle
    g = torch.Generator().manual_seed(11)
    B, H, dqk, dv = 2, 3, 8, 5
    z = torch.zeros
    q, k, v = z(B, H, 0, dqk), z(B, H, 0, dqk), z(B, H, 0, dv)
    i_pre = f_pre = z(B, H, 0)
    C0, n0, m0 = torch.randn(B, H, dqk, dv, generator=g), torch.randn(B, H, dqk, generator=g), \
        torch.randn(B, H, generator=g)
    h, C1, n1, m1 = oracle.recurrent(q, k, v, i_pre, f_pre, None, C0, n0, m0)
    assert h.shape == (B, H, 0, dv)
    np.testing.assert_array_equal(C1, C0.double().numpy())
    np.testing.assert_array_equal(n1, n0.double().numpy())
    np.testing.assert_array_equal(m1, m0.double().numpy())
    dC1, dn1 = torch.randn(B, H, dqk, dv, generator=g), torch.randn(B, H, dqk, generator=g)
    r = oracle.backward(q, k, v, i_pre, f_pre, None, C0, n0, m0, z(B, H, 0, dv), dC1, dn1)
    np.testing.assert_allclose(r["dC0"], dC1.double().numpy(), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(r["dn0"], dn1.double().numpy(), rtol=1e-13, atol=1e-13)
    ref = (dC1.double() * C0.double()).sum((2, 3)) + (dn1.double() * n0.double()).sum(2)
    np.testing.assert_allclose(r["dm0"], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_given_h_equal_to_own_h_changes_nothing():
    """Handing the oracle its own fp64 forward output as h gives the same
    gradients as leaving h out (the two h-dependent terms are the same
    numbers, computed from the given h instead of num/den)."""
    c = make_case(21, T=70, o=True, state=True, dstate=True)
    h, *_ = oracle.recurrent(c["q"], c["k"], c["v"], c["i_pre"], c["f_pre"], c["o_pre"],
                             c["C0"], c["n0"], c["m0"])
    g0 = grads(c, "sigmoid")
    g1 = oracle.backward(c["q"], c["k"], c["v"], c["i_pre"], c["f_pre"], c["o_pre"], c["C0"],
                         c["n0"], c["m0"], c["dh"], c["dC1"], c["dn1"], h=h)
    for name in ("dq", "dk", "dv", "di", "df", "do", "dC0", "dn0", "dm0"):
        np.testing.assert_allclose(g1[name], g0[name], rtol=1e-12, atol=1e-13, err_msg=name)


def test_given_h_single_token_closed_form():
    """One token from the zero state on the active branch (|i q.k| = 4), with a
    given output h' = sign(q.k) v + delta instead of the exact sign(q.k) v.
    The denominator term is dnq = -s (dh . h') / den with s = sign(q.k) and
    den = i |q.k|, so dq = i k (v . dh - s dh . h') / den = -k s (dh . delta) /
    |q.k| and dk likewise with q; the exact h gives zero.  With an o-gate,
    do~ = dh (.) h' (.) (1 - sigmoid(o~))."""
    rng = np.random.default_rng(13)
    dqk, dv = 5, 3
    q = rng.normal(0, 1, dqk)
    k = rng.normal(0, 1, dqk) / np.sqrt(dqk)
    v = rng.normal(0, 1, dv)
    dh = rng.normal(0, 1, dv)
    delta = rng.normal(0, 0.01, dv)
    qk = q @ k
    s = np.sign(qk)
    ip = np.log(4.0 / abs(qk))
    e = lambda a: np.asarray(a, dtype=np.float64).reshape((1, 1, 1) + np.shape(a))  # noqa: E731
    g = oracle.backward(e(q), e(k), e(v), e(ip), e(1.0), None, None, None, None, e(dh),
                        h=e(s * v + delta))
    np.testing.assert_allclose(g["dq"].reshape(-1), -k * s * (dh @ delta) / abs(qk),
                               rtol=1e-11, atol=1e-15)
    np.testing.assert_allclose(g["dk"].reshape(-1), -q * s * (dh @ delta) / abs(qk),
                               rtol=1e-11, atol=1e-15)
    o = rng.normal(0, 1, dv)
    sig = 1.0 / (1.0 + np.exp(-o))
    hp = s * sig * v + delta
    g = oracle.backward(e(q), e(k), e(v), e(ip), e(1.0), e(o), None, None, None, e(dh), h=e(hp))
    np.testing.assert_allclose(g["do"].reshape(-1), dh * hp * (1 - sig), rtol=1e-13, atol=0)


def test_conditioning_single_token_closed_form():
    """One token on the active branch with the exact h: the memory and
    normalizer paths of dq, dk and di cancel exactly (the results are 0,
    test_single_token_closed_form), and the conditioning scale is the sum of
    their sizes: cond_dq = 2 |k| |v . dh| / |q.k|, cond_dk = 2 |q| |v . dh| /
    |q.k|, cond_di = 2 |v . dh|."""
    rng = np.random.default_rng(17)
    dqk, dv = 4, 6
    q = rng.normal(0, 1, dqk)
    k = rng.normal(0, 1, dqk) / np.sqrt(dqk)
    v = rng.normal(0, 1, dv)
    dh = rng.normal(0, 1, dv)
    qk = q @ k
    ip = np.log(3.0 / abs(qk))
    e = lambda a: np.asarray(a, dtype=np.float64).reshape((1, 1, 1) + np.shape(a))  # noqa: E731
    g = oracle.backward(e(q), e(k), e(v), e(ip), e(1.0), None, None, None, None, e(dh))
    vd = abs(v @ dh)
    np.testing.assert_allclose(g["cond_dq"].reshape(-1), 2 * np.abs(k) * vd / abs(qk), rtol=1e-12)
    np.testing.assert_allclose(g["cond_dk"].reshape(-1), 2 * np.abs(q) * vd / abs(qk), rtol=1e-12)
    np.testing.assert_allclose(g["cond_di"].item(), 2 * vd, rtol=1e-12)


def test_conditioning_bounds_and_linear_attention():
    """cond >= |gradient| always (triangle inequality), and with no active
    denominator anywhere (causal linear attention, |n.q| < 1) the normalizer
    paths vanish, so cond equals |gradient| exactly."""
    c = make_case(23, T=70, o=True, state=True, dstate=True)
    g = grads(c, "sigmoid")
    for name in ("dq", "dk", "di", "df", "dm0"):
        assert np.all(g["cond_" + name] >= np.abs(g[name]) * (1 - 1e-12) - 1e-300), name
    rng = np.random.default_rng(5)
    T, dqk, dv = 40, 6, 4
    q = rng.normal(0, 1, (T, dqk)) * 0.1
    k = rng.normal(0, 1, (T, dqk)) * 0.1 / np.sqrt(dqk)
    v = rng.normal(0, 1, (T, dv))
    dh = rng.normal(0, 1, (T, dv))
    e = lambda a: np.asarray(a, dtype=np.float64)[None, None]  # noqa: E731
    g = oracle.backward(e(q), e(k), e(v), e(np.zeros(T)), e(np.zeros(T)), None, None, None, None,
                        e(dh), fgate="exp")
    for name in ("dq", "dk", "di", "df"):
        np.testing.assert_allclose(g["cond_" + name], np.abs(g[name]), rtol=1e-12, atol=1e-300,
                                   err_msg=name)
