"""Write the exact-rational golden fixtures under tests/golden/.

The pages print no worked numeric example, so these fixtures are produced by
the exact rational oracle (oracle/exact.py) on small hand-chosen rational
inputs. Run from the repository root:  python tests/golden/make_golden.py
The fixtures guard the fp64 oracle against regressions; their pin is the
exact arithmetic plus the transition-product unrolling checked in
tests/test_oracle_pins.py.
"""
import json
import os
import sys
from fractions import Fraction

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(
    os.path.abspath(__file__)))))
from oracle import exact as X  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))


def s(x):
    if isinstance(x, list):
        return [s(e) for e in x]
    return str(Fraction(x))


def osdn_case():
    F = Fraction
    q = [[1, 0, F(1, 2)], [0, 1, 0], [F(1, 2), F(1, 2), F(1, 2)], [1, -1, 0]]
    k = [[F(1, 2), F(1, 2), 0], [0, F(3, 4), F(1, 4)], [F(1, 2), 0, F(-1, 2)],
         [F(1, 4), F(1, 4), F(1, 2)]]
    v = [[1, 2], [-1, F(1, 2)], [F(3, 2), 0], [0, -2]]
    beta = [F(1, 2), F(3, 4), F(1, 4), F(1, 2)]
    r = [1, F(7, 8), F(3, 4), 1]
    eta = F(1, 10)
    d0 = [1, 1, 1]
    S0 = [[0, 0, 0], [0, 0, 0]]
    o, S, d, ktil, _ = X.osdn_exact(q, k, v, beta, r, eta, d0, S0)
    return dict(
        citation=("OSDN token recurrence: [OSDN-it] sections 2.1 (update with "
                  "k~ = d*k), 2.2 (closed-form surrogate), 2.3 (forgetting "
                  "gate, descent sign); inclusive readout o_t = S_t q_t."),
        inputs=dict(q=s(q), k=s(k), v=s(v), beta=s(beta), r=s(r), eta=s(eta),
                    d0=s(d0), S0=s(S0)),
        expected=dict(o=s(o), S_T=s(S), d_T=s(d), ktilde=s(ktil)))


def gdn2_case():
    F = Fraction
    q = [[1, 0, 1], [0, 1, 0], [1, 1, 0]]
    k = [[F(1, 2), F(1, 2), 0], [0, 1, 0], [F(1, 2), 0, F(1, 2)]]
    v = [[1, -1], [2, 0], [0, 1]]
    alpha = [[1, F(1, 2), F(3, 4)], [F(7, 8), 1, 1], [F(1, 2), F(1, 2), 1]]
    b = [[1, F(1, 2), 0], [F(1, 4), 1, F(1, 2)], [F(1, 2), F(1, 2), F(1, 2)]]
    w = [[1, F(1, 2)], [F(3, 4), 1], [F(1, 2), F(1, 4)]]
    S0 = [[1, 0], [0, 1], [F(1, 2), F(-1, 2)]]
    o, S, _ = X.gdn2_exact(q, k, v, alpha, b, w, S0)
    return dict(
        citation=("Gated DeltaNet-2 recurrence: [GDN2-it] method part 1 (erase "
                  "and write gates, per-channel decay); read orientation from "
                  "method part 2; output o_t = S_t^T q_t."),
        inputs=dict(q=s(q), k=s(k), v=s(v), alpha=s(alpha), b=s(b), w=s(w),
                    S0=s(S0)),
        expected=dict(o=s(o), S_T=s(S)))


if __name__ == "__main__":
    for name, case in [("osdn_tiny_exact.json", osdn_case()),
                       ("gdn2_tiny_exact.json", gdn2_case())]:
        with open(os.path.join(HERE, name), "w") as f:
            json.dump(case, f, indent=1)
        print("wrote", name)
