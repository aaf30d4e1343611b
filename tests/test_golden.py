"""fp64 oracle against the exact-rational golden fixtures in tests/golden/."""
import json
import os
from fractions import Fraction

import numpy as np

from oracle import recurrence as R

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(HERE, name)) as f:
        case = json.load(f)

    def num(x):
        a = np.vectorize(lambda s: float(Fraction(s)))(np.array(x, dtype=object))
        return a.astype(np.float64)

    return case, num


def test_osdn_golden():
    case, num = _load("osdn_tiny_exact.json")
    i, e = case["inputs"], case["expected"]
    o, S, d, tr = R.osdn_ref(num(i["q"])[None, None], num(i["k"])[None, None],
                             num(i["v"])[None, None], num(i["beta"])[None, None],
                             num(i["r"])[None, None], float(Fraction(i["eta"])),
                             num(i["d0"])[None, None], num(i["S0"])[None, None],
                             return_trace=True)
    np.testing.assert_allclose(o[0, 0], num(e["o"]), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(S[0, 0], num(e["S_T"]), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(d[0, 0], num(e["d_T"]), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(tr["ktilde"][0, 0], num(e["ktilde"]),
                               rtol=1e-13, atol=1e-15)


def test_gdn2_golden():
    case, num = _load("gdn2_tiny_exact.json")
    i, e = case["inputs"], case["expected"]
    o, S = R.gdn2_ref(num(i["q"])[None, None], num(i["k"])[None, None],
                      num(i["v"])[None, None],
                      np.log(num(i["alpha"]))[None, None],
                      num(i["b"])[None, None], num(i["w"])[None, None],
                      num(i["S0"])[None, None])
    np.testing.assert_allclose(o[0, 0], num(e["o"]), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(S[0, 0], num(e["S_T"]), rtol=1e-13, atol=1e-15)
