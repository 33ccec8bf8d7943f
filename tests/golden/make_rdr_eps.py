"""Writes tests/golden/rdr_eps_d128.txt: the angular error eps(b) of ADA's
estimator at d = 128, the distortion surrogate of the RDR controller (section
2.2 of the page: the logit error is dominated by the angular approximation
error, scaled by the query and key magnitudes).

eps(b) = RMS over random pairs of unit vectors (q, k) of
    f_b(c_q, c_k) - <q, k>,   f_b = <u(centres(c_q)), u(centres(c_k))>,
both directions coded at b bits, computed with the oracle only.  Keys are
N(0, 1) (uniform directions), 2000 pairs per width, seed 20260609.

    python tests/golden/make_rdr_eps.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
from oracle import oracle as O  # noqa: E402

D, PAIRS, SEED = 128, 2000, 20260609


def eps_table():
    rng = np.random.default_rng(SEED)
    q = rng.standard_normal((PAIRS, D)).astype(np.float32)
    k = rng.standard_normal((PAIRS, D)).astype(np.float32)
    out = {}
    for b in (2, 3, 4, 6, 8):
        err = np.empty(PAIRS)
        for i in range(PAIRS):
            uq = O.direction(O.key_codes(q[i], b)[0], D, b)
            uk = O.direction(O.key_codes(k[i], b)[0], D, b)
            qd, kd = q[i].astype(np.float64), k[i].astype(np.float64)
            err[i] = uq @ uk - (qd @ kd) / (np.linalg.norm(qd) * np.linalg.norm(kd))
        out[b] = float(np.sqrt(np.mean(err * err)))
    return out


if __name__ == "__main__":
    t = eps_table()
    with open(os.path.join(HERE, "rdr_eps_d128.txt"), "w") as f:
        f.write("# RMS of f_b(c_q, c_k) - <q, k> over %d random unit pairs, d = %d, seed %d\n" % (PAIRS, D, SEED))
        f.write("# written by tests/golden/make_rdr_eps.py (oracle only)\n")
        for b, e in t.items():
            f.write("%d %.6e\n" % (b, e))
    print(open(os.path.join(HERE, "rdr_eps_d128.txt")).read())
