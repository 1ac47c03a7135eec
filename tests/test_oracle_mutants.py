"""The oracle's pins are discriminating: plant one plausible mistake at a time in
a copy of the oracle's C source (on the CPU), rebuild it, and check that at
least one pin rejects the mutant.  The real oracle passes the same checks.
"""
from __future__ import annotations

import math
import os

import numpy as np
import pytest

import oracle
from oracle import unrolled_mp
from test_oracle import (BRUTE_CASES, mp_to_np, np_logsigmoid, quadratic_form,
                         rel_err, tiny_case, to_lists)

# (name, original text, planted mistake)
MUTANTS = [
    ("abs dropped from the denominator",
     "dmax(fabs(nq), exp(-m_new))", "dmax(nq, exp(-m_new))"),
    ("denominator floor dropped",
     "dmax(fabs(nq), exp(-m_new))", "fabs(nq)"),
    ("sigmoid forget gate taken as exponential",
     "? logsigmoid(f_pre) : f_pre", "? f_pre : f_pre"),
    ("readout of C transposed",
     "num += q[a] * C[a * dv + b]", "num += q[a] * C[b * dqk + a]"),
    ("input-gate exponent sign flipped",
     "exp(i_pre - m_new)", "exp(m_new - i_pre)"),
    ("normalizer decay dropped",
     "n[a] = fp * n[a] + ika", "n[a] = n[a] + ika"),
    ("output gate applied without sigmoid",
     "o ? sigmoid(o[b]) : 1.0", "o ? o[b] : 1.0"),
    ("running maximum ignores the forget gate",
     "dmax(lf + *m, i_pre)", "dmax(*m, i_pre)"),
    ("value and key swapped in the memory update",
     "row[b] = fp * row[b] + ika * v[b]", "row[b] = fp * row[b] + ip * v[a % dv] * k[b % dqk]"),
    # edited by _exclusive_readout below (a move, not a text swap)
    ("readout before the token's own update (exclusive)", None, None),
]


def _exclusive_readout(src: str) -> str:
    """Move the memory update after the readout: h_t then reads C_{t-1}."""
    upd_start = src.index("  for (int64_t a = 0; a < dqk; ++a) {\n    double ika")
    upd_end = src.index("  *m = m_new;")
    update = src[upd_start:upd_end]
    src = src[:upd_start] + src[upd_end:]
    body_end = src.index("    h[b] = gate * num / den;\n  }\n") + len("    h[b] = gate * num / den;\n  }\n")
    return src[:body_end] + update + src[body_end:]


def pins_pass(lib) -> bool:
    """A compact run of the pins: brute force, closed-form maximum, quadratic
    form, linear attention.  True when every check passes."""
    try:
        for seed, T, dqk, dv, fgate, state, o in BRUTE_CASES:
            f_dist = (1.0, 1.0) if fgate == "sigmoid" else (-0.3, 0.5)
            c = tiny_case(seed, T, dqk, dv, fgate=fgate, state=state, o=o, f_dist=f_dist)
            e4 = lambda a: None if a is None else np.asarray(a)[None, None]  # noqa: E731
            m0 = None if c["m0"] is None else np.array([[c["m0"]]])
            h, C1, n1, m1 = oracle.recurrent(e4(c["q"]), e4(c["k"]), e4(c["v"]),
                                             e4(c["i_pre"]), e4(c["f_pre"]), e4(c["o_pre"]),
                                             e4(c["C0"]), e4(c["n0"]), m0, fgate=fgate, lib=lib)
            hb, Cb, nb = unrolled_mp.unrolled(**to_lists(c), fgate=fgate)
            if not (rel_err(h[0, 0], mp_to_np(hb)) < 1e-13):
                return False
            if not (rel_err(C1[0, 0] * math.exp(m1[0, 0]), mp_to_np(Cb)) < 1e-13):
                return False
            if not (rel_err(n1[0, 0] * math.exp(m1[0, 0]), mp_to_np(nb)) < 1e-13):
                return False
        # closed-form running maximum
        rng = np.random.default_rng(7)
        T = 60
        ip = rng.normal(-2, 3, T)
        fp = rng.normal(1, 2, T)
        c = tiny_case(8, T, 3, 3, state=True)
        c.update(i_pre=ip, f_pre=fp)
        e4 = lambda a: None if a is None else np.asarray(a)[None, None]  # noqa: E731
        _, _, _, m1 = oracle.recurrent(e4(c["q"]), e4(c["k"]), e4(c["v"]), e4(ip), e4(fp),
                                       None, e4(c["C0"]), e4(c["n0"]),
                                       np.array([[c["m0"]]]), lib=lib)
        F = np.cumsum(np_logsigmoid(fp))
        mt = F[-1] + max(c["m0"], np.max(ip - F))
        if not abs(m1[0, 0] - mt) < 1e-12:
            return False
        # quadratic form
        c = tiny_case(21, 80, 5, 7, state=True, i_dist=(0.0, 2.0), f_dist=(2.0, 1.0))
        h, C1, n1, m1 = oracle.recurrent(e4(c["q"]), e4(c["k"]), e4(c["v"]), e4(c["i_pre"]),
                                         e4(c["f_pre"]), e4(c["o_pre"]), e4(c["C0"]),
                                         e4(c["n0"]), np.array([[c["m0"]]]), lib=lib)
        hq, Cq, nq, mq = quadratic_form(c["q"], c["k"], c["v"], c["i_pre"], c["f_pre"],
                                        c["o_pre"], c["C0"], c["n0"], c["m0"], "sigmoid")
        if not (rel_err(h[0, 0], hq) < 1e-10 and rel_err(C1[0, 0], Cq) < 1e-10):
            return False
        return True
    except (AssertionError, ValueError, FloatingPointError):
        return False


def test_real_oracle_passes_compact_pins():
    assert pins_pass(None)


@pytest.mark.parametrize("name,orig,mut", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, orig, mut):
    src = oracle.source_text()
    if name.startswith("readout before"):
        bad = _exclusive_readout(src)
    else:
        assert orig in src, f"mutation anchor not found: {orig!r}"
        bad = src.replace(orig, mut)
    assert bad != src
    path = oracle.build_variant(bad, os.path.join(str(tmp_path), "libmutant.so"))
    lib = oracle.load_library(path)
    assert not pins_pass(lib), f"pins did not catch: {name}"
