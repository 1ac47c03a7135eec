"""Brute-force evaluation of the mLSTM cell from its unrolled sums, in mpmath.

TEST INFRASTRUCTURE ONLY (a pin for the fp64 recurrence in ``mlstm_oracle.c``).

Source: the xLSTM post (llms.blog), section 3, sub-section "The Parallel Dual
Form": unrolling the matrix update from the first token gives the memory at
step t as a sum over earlier tokens s of (product of the forget gates after s)
times i_s v_s k_s^T, and the retrieval C_t q_t as the same sum with the scalar
(q_t . k_s).  The normalizer n_t unrolls the same way with k_s in place of
v_s k_s^T (sub-section "Associative Matrix Cell State").  The retrieval is
C_t q_t / max(|n_t . q_t|, 1) gated by sigmoid(o~_t).

Nothing here is stabilized and nothing is recursive: every C_t and n_t is
summed afresh from token 1, in 50-digit arithmetic, so a mistake in the
recurrence's stabilizer, orientation, gating or denominator shows up as a
mismatch.  Only usable on tiny inputs (T <= ~16, d <= ~6).

Orientation: C is returned as [d_qk][d_v] (the transpose of the page's
v k^T), matching the oracle's storage.  An initial stabilized state
(C~_0, n~_0, m_0) contributes (product of all forget gates up to t) times the
true initial memory C~_0 e^{m_0}.
"""
from __future__ import annotations

import mpmath as mp

DIGITS = 50


def _gate_f(fpre, fgate):
    fpre = mp.mpf(fpre)
    if fgate == "sigmoid":
        return 1 / (1 + mp.exp(-fpre))
    if fgate == "exp":
        return mp.exp(fpre)
    raise ValueError(fgate)


def unrolled(q, k, v, i_pre, f_pre, o_pre=None, C0=None, n0=None, m0=None,
             fgate="sigmoid"):
    """One head.  q, k: T x dqk; v: T x dv; i_pre, f_pre: T; o_pre: T x dv or
    None; C0: dqk x dv, n0: dqk, m0: scalar, or None (zero memory).

    All inputs are nested Python sequences of floats (exact binary values).
    Returns (h, C_T, n_T) as nested lists of mpmath numbers, where C_T and
    n_T are the TRUE (unstabilized) memory and normalizer after the last token.
    """
    with mp.workdps(DIGITS):
        T = len(q)
        dqk = len(q[0])
        dv = len(v[0])
        f = [_gate_f(f_pre[t], fgate) for t in range(T)]
        ig = [mp.exp(mp.mpf(i_pre[t])) for t in range(T)]

        def decay(s, t):
            """product of f_tau for tau = s+1 .. t (0-based tokens s < tau <= t)"""
            p = mp.mpf(1)
            for tau in range(s + 1, t + 1):
                p *= f[tau]
            return p

        if C0 is not None:
            scale0 = mp.exp(mp.mpf(m0))
            Ctrue0 = [[mp.mpf(C0[a][b]) * scale0 for b in range(dv)] for a in range(dqk)]
            ntrue0 = [mp.mpf(n0[a]) * scale0 for a in range(dqk)]
        else:
            Ctrue0 = [[mp.mpf(0)] * dv for _ in range(dqk)]
            ntrue0 = [mp.mpf(0)] * dqk

        h = []
        C_t = n_t = None
        for t in range(T):
            # decay of the initial memory over tokens 0..t
            d0 = decay(-1, t)
            C_t = [[d0 * Ctrue0[a][b] for b in range(dv)] for a in range(dqk)]
            n_t = [d0 * ntrue0[a] for a in range(dqk)]
            for s in range(t + 1):
                w = decay(s, t) * ig[s]
                for a in range(dqk):
                    ka = mp.mpf(k[s][a])
                    n_t[a] += w * ka
                    for b in range(dv):
                        C_t[a][b] += w * ka * mp.mpf(v[s][b])
            nq = mp.fsum(n_t[a] * mp.mpf(q[t][a]) for a in range(dqk))
            den = max(abs(nq), mp.mpf(1))
            row = []
            for b in range(dv):
                num = mp.fsum(mp.mpf(q[t][a]) * C_t[a][b] for a in range(dqk))
                gate = 1 / (1 + mp.exp(-mp.mpf(o_pre[t][b]))) if o_pre is not None else mp.mpf(1)
                row.append(gate * num / den)
            h.append(row)
        return h, C_t, n_t


def retrieval_terms(q, k, v, i_pre, f_pre, C0=None, n0=None, m0=None,
                    fgate="sigmoid"):
    """The unstabilized n_t . q_t for every token (to check that a test input
    exercises both branches of max(|n.q|, 1))."""
    with mp.workdps(DIGITS):
        T = len(q)
        out = []
        for t in range(T):
            _, _, n_t = unrolled(q[: t + 1], k[: t + 1], v[: t + 1], i_pre[: t + 1],
                                 f_pre[: t + 1], None, C0, n0, m0, fgate)
            out.append(mp.fsum(n_t[a] * mp.mpf(q[t][a]) for a in range(len(q[0]))))
        return out
