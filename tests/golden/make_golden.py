"""Writes the golden fixtures in this folder.  Calls only ``oracle.unrolled_mp``.

The pages print no worked numeric example of the mLSTM cell, so the stored
values come from the unrolled-sum form of the xLSTM post (section 3, "The
Parallel Dual Form": the memory as a decayed sum of i_s v_s k_s^T; "Associative
Matrix Cell State": retrieval C_t q_t / max(|n_t . q_t|, 1), gated by
sigmoid(o~_t)), evaluated in 50-digit arithmetic with no stabilizer.

Run from the repository root:  python tests/golden/make_golden.py
"""
from __future__ import annotations

import json
import os
import random
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import unrolled_mp  # noqa: E402

CITATION = ("xLSTM post (llms.blog), section 3: 'The Parallel Dual Form' (unrolled "
            "sum of the memory) and 'Associative Matrix Cell State' (retrieval "
            "with max(|n.q|, 1), output gate)")


def _draw(rnd: random.Random, shape, mean, std):
    if len(shape) == 1:
        return [rnd.gauss(mean, std) for _ in range(shape[0])]
    return [_draw(rnd, shape[1:], mean, std) for _ in range(shape[0])]


def case(name, seed, T, dqk, dv, fgate, with_state, with_o, i_dist, f_dist):
    rnd = random.Random(seed)
    q = _draw(rnd, (T, dqk), 0.0, 1.0)
    k = _draw(rnd, (T, dqk), 0.0, 1.0)
    v = _draw(rnd, (T, dv), 0.0, 1.0)
    i_pre = _draw(rnd, (T,), *i_dist)
    f_pre = _draw(rnd, (T,), *f_dist)
    o_pre = _draw(rnd, (T, dv), 0.0, 1.0) if with_o else None
    C0 = n0 = m0 = None
    if with_state:
        C0 = _draw(rnd, (dqk, dv), 0.0, 1.0)
        n0 = _draw(rnd, (dqk,), 0.0, 1.0)
        m0 = rnd.gauss(0.0, 1.0)
    h, C, n = unrolled_mp.unrolled(q, k, v, i_pre, f_pre, o_pre, C0, n0, m0, fgate)
    return {
        "name": name, "citation": CITATION, "fgate": fgate,
        "T": T, "dqk": dqk, "dv": dv,
        "inputs": {"q": q, "k": k, "v": v, "i_pre": i_pre, "f_pre": f_pre,
                   "o_pre": o_pre, "C0": C0, "n0": n0, "m0": m0},
        "expected": {
            "h": [[float(x) for x in row] for row in h],
            "C_true": [[float(x) for x in row] for row in C],
            "n_true": [float(x) for x in n],
        },
    }


def main():
    cases = [
        case("sigmoid_zero_state_gated", 11, 7, 3, 4, "sigmoid", False, True, (0.5, 1.0), (1.0, 1.0)),
        case("sigmoid_random_state", 12, 8, 4, 3, "sigmoid", True, False, (0.5, 1.0), (1.0, 1.0)),
        case("exp_random_state_gated", 13, 6, 2, 5, "exp", True, True, (0.3, 1.0), (-0.3, 0.5)),
    ]
    out = os.path.join(HERE, "unrolled_small.json")
    with open(out, "w") as fh:
        json.dump({"source": CITATION, "digits": unrolled_mp.DIGITS, "cases": cases}, fh,
                  indent=1)
    print("wrote", out)


if __name__ == "__main__":
    main()
