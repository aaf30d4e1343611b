"""Pins of the oracle's backward pass (oracle/backward.py) against central
differences of the forward oracle osdn_ref: the adjoint must be the gradient
of L = <do, o> + <dS_T, S_T> + <dd_T, d_T> for every input, including the
preconditioner learner's (phase 1: k, beta, r, eta, d0). Planted mistakes in
the adjoint are caught."""
import numpy as np
import pytest

from oracle import backward as BW
from oracle import recurrence as R


def _case(seed, B=1, H=2, T=9, Dk=5, Dv=4, unit=False):
    g = np.random.default_rng(seed)
    k = g.standard_normal((B, H, T, Dk))
    if unit:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    x = dict(q=g.standard_normal((B, H, T, Dk)), k=k,
             v=g.standard_normal((B, H, T, Dv)),
             beta=g.uniform(0.1, 0.9, (B, H, T)),
             r=g.uniform(0.6, 1.0, (B, H, T)), eta=0.3,
             d0=g.uniform(0.5, 1.5, (B, H, Dk)),
             S0=0.5 * g.standard_normal((B, H, Dv, Dk)))
    adj = dict(do=g.standard_normal((B, H, T, Dv)),
               dS_T=g.standard_normal((B, H, Dv, Dk)),
               dd_T=g.standard_normal((B, H, Dk)))
    return x, adj


def _loss(x, adj, scale=1.0):
    o, S, d = R.osdn_ref(x["q"], x["k"], x["v"], x["beta"], x["r"], x["eta"],
                         x["d0"], x["S0"], scale)
    return (np.sum(adj["do"] * o) + np.sum(adj["dS_T"] * S)
            + np.sum(adj["dd_T"] * d))


def pin_backward_matches_central_differences(backward=None):
    """Every gradient, element by element, against central differences of
    the forward oracle (fp64, h = 1e-6)."""
    backward = backward or BW.osdn_backward_ref
    x, adj = _case(3)
    scale = 0.7
    gr = backward(x["q"], x["k"], x["v"], x["beta"], x["r"], x["eta"], x["d0"],
                  x["S0"], adj["do"], adj["dS_T"], adj["dd_T"], scale)
    h = 1e-6
    for name in ("q", "k", "v", "beta", "r", "d0", "S0"):
        a = x[name]
        num = np.zeros_like(a)
        for idx in np.ndindex(a.shape):
            xp = dict(x); xm = dict(x)
            ap, am = a.copy(), a.copy()
            ap[idx] += h
            am[idx] -= h
            xp[name], xm[name] = ap, am
            num[idx] = (_loss(xp, adj, scale) - _loss(xm, adj, scale)) / (2 * h)
        np.testing.assert_allclose(gr[name], num, rtol=1e-6, atol=1e-7,
                                   err_msg=name)
    xp = dict(x); xm = dict(x)
    xp["eta"], xm["eta"] = x["eta"] + h, x["eta"] - h
    num = (_loss(xp, adj, scale) - _loss(xm, adj, scale)) / (2 * h)
    np.testing.assert_allclose(gr["eta"].sum(), num, rtol=1e-6, atol=1e-7)


def test_backward_matches_central_differences():
    pin_backward_matches_central_differences()


def test_backward_zero_key_and_unit_keys():
    """A zero key row (no step there, no gradient through g) and unit keys,
    against directional central differences on every input at once."""
    x, adj = _case(4, T=12, Dk=6, Dv=3, unit=True)
    x["k"][0, 1, 5] = 0.0
    gr = BW.osdn_backward_ref(x["q"], x["k"], x["v"], x["beta"], x["r"],
                              x["eta"], x["d0"], x["S0"], adj["do"], adj["dS_T"],
                              adj["dd_T"])
    g = np.random.default_rng(5)
    dirs = {n: g.standard_normal(np.shape(x[n])) for n in
            ("q", "v", "beta", "r", "d0", "S0")}
    dirs["k"] = g.standard_normal(x["k"].shape)
    dirs["k"][0, 1, 5] = 0.0   # stay on the zero row (the convention's kink)
    h = 1e-6
    xp = {n: (x[n] + h * dirs[n] if n in dirs else x[n]) for n in x}
    xm = {n: (x[n] - h * dirs[n] if n in dirs else x[n]) for n in x}
    num = (_loss(xp, adj) - _loss(xm, adj)) / (2 * h)
    ana = sum(np.sum(gr[n] * dirs[n]) for n in dirs)
    assert abs(num - ana) <= 1e-6 * max(1.0, abs(num))


def test_backward_without_gate_and_defaults():
    """r, d0, S0 left at their defaults (ones, ones, zeros) and no final
    adjoints: the result equals the explicit call."""
    x, adj = _case(6)
    B, H, T, Dk = x["k"].shape
    Dv = x["v"].shape[-1]
    a = BW.osdn_backward_ref(x["q"], x["k"], x["v"], x["beta"], None, 0.2, None,
                             None, adj["do"])
    b = BW.osdn_backward_ref(x["q"], x["k"], x["v"], x["beta"],
                             np.ones((B, H, T)), 0.2, np.ones((B, H, Dk)),
                             np.zeros((B, H, Dv, Dk)), adj["do"],
                             np.zeros((B, H, Dv, Dk)), np.zeros((B, H, Dk)))
    for n in a:
        np.testing.assert_allclose(a[n], b[n], rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------------------
# planted mistakes in the adjoint
# ---------------------------------------------------------------------------

def _mutant(edit):
    src = open(BW.__file__).read()
    assert edit[0] in src, edit[0]
    ns = {}
    code = src.replace(edit[0], edit[1])
    code = code.replace("from .recurrence import _f64", "from oracle.recurrence import _f64")
    exec(compile(code, "mutant", "exec"), ns)
    return ns["osdn_backward_ref"]


MUTANTS = [
    ("dk = -bt[..., None] * np.einsum", "dk = 0.0 * np.einsum"),          # drop the read-key path
    ("dd_t = dd_t + rt[..., None] * dd", "dd_t = dd_t + dd"),            # forget the gate in the d adjoint
    ("dc = np.where(live, -eta * bt * bt", "dc = np.where(live, eta * bt * bt"),  # sign of dc
    ("da = da + dc[..., None] * d_t + dn[..., None]", "da = da + dc[..., None] * d_t"),  # drop dn
    ("dS_prev = dS - bt[..., None, None] * w[..., :, None] * kt[..., None, :]",
     "dS_prev = dS - bt[..., None, None] * w[..., :, None] * kt_[..., None, :]"),  # k~ for k
    ("dS = dS + scale * do[..., t, :, None]", "dS = dS + do[..., t, :, None]"),  # drop scale
]


@pytest.mark.parametrize("edit", MUTANTS, ids=[m[1][:30] for m in MUTANTS])
def test_backward_mutants_are_caught(edit):
    with pytest.raises(AssertionError):
        pin_backward_matches_central_differences(_mutant(edit))
