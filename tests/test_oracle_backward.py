"""Pins of the oracle's backward passes (oracle/backward.py) against central
differences of the forward oracles: each adjoint must be the gradient of
L = <do, o> + <dS_T, S_T> (+ <dd_T, d_T>) for every input, including the
preconditioner learner's (phase 1: k, beta, r, eta, d0) and, in the
gate-aware adjoints of OSDN on a decaying backbone (osdn_gated_ref) and of
GDN-2 (gdn2_ref), the decay and the erase and write gates. Planted mistakes
in each adjoint are caught."""
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


# ---------------------------------------------------------------------------
# gate-aware adjoints: OSDN on a per-channel-decay backbone, and GDN-2
# ---------------------------------------------------------------------------

def _numeric_grads(loss, x, names, h=1e-6):
    out = {}
    for name in names:
        a = x[name]
        num = np.zeros_like(a)
        for idx in np.ndindex(a.shape):
            xp = dict(x); xm = dict(x)
            ap, am = a.copy(), a.copy()
            ap[idx] += h
            am[idx] -= h
            xp[name], xm[name] = ap, am
            num[idx] = (loss(xp) - loss(xm)) / (2 * h)
        out[name] = num
    return out


def _gated_case(seed):
    x, adj = _case(seed, T=8, Dk=4, Dv=3)
    g = np.random.default_rng(seed + 100)
    x["log_alpha"] = -g.uniform(0.05, 1.5, x["k"].shape)
    return x, adj


def _gated_loss(adj, scale):
    def loss(x):
        o, S, d = R.osdn_gated_ref(x["q"], x["k"], x["v"], x["beta"],
                                   x["log_alpha"], x["r"], x["eta"], x["d0"],
                                   x["S0"], scale)
        return (np.sum(adj["do"] * o) + np.sum(adj["dS_T"] * S)
                + np.sum(adj["dd_T"] * d))
    return loss


def pin_gated_backward(backward=None):
    """osdn_gated_backward_ref, every gradient element by element, against
    central differences of osdn_gated_ref."""
    backward = backward or BW.osdn_gated_backward_ref
    x, adj = _gated_case(7)
    scale = 0.8
    gr = backward(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], x["r"],
                  x["eta"], x["d0"], x["S0"], adj["do"], adj["dS_T"],
                  adj["dd_T"], scale)
    loss = _gated_loss(adj, scale)
    names = ("q", "k", "v", "beta", "log_alpha", "r", "d0", "S0")
    num = _numeric_grads(loss, x, names)
    for name in names:
        np.testing.assert_allclose(gr[name], num[name], rtol=1e-6, atol=1e-7,
                                   err_msg=name)
    h = 1e-6
    xp = dict(x); xm = dict(x)
    xp["eta"], xm["eta"] = x["eta"] + h, x["eta"] - h
    np.testing.assert_allclose(gr["eta"].sum(), (loss(xp) - loss(xm)) / (2 * h),
                               rtol=1e-6, atol=1e-7)


def test_gated_backward_matches_central_differences():
    pin_gated_backward()


def test_gated_backward_without_decay_is_the_plain_adjoint():
    """log alpha = 0 everywhere: the gated adjoint equals osdn_backward_ref,
    and log alpha's gradient is then sum_i dS_{t-1}[i, j] S_{t-1}[i, j]."""
    x, adj = _case(8)
    zero = np.zeros(x["k"].shape)
    a = BW.osdn_gated_backward_ref(x["q"], x["k"], x["v"], x["beta"], zero,
                                   x["r"], x["eta"], x["d0"], x["S0"],
                                   adj["do"], adj["dS_T"], adj["dd_T"])
    b = BW.osdn_backward_ref(x["q"], x["k"], x["v"], x["beta"], x["r"],
                             x["eta"], x["d0"], x["S0"], adj["do"],
                             adj["dS_T"], adj["dd_T"])
    for n in b:
        np.testing.assert_allclose(a[n], b[n], rtol=1e-13, atol=1e-13)


def _gdn2_case(seed, B=1, H=2, T=8, Dk=4, Dv=3):
    g = np.random.default_rng(seed)
    x = dict(q=g.standard_normal((B, H, T, Dk)),
             k=g.standard_normal((B, H, T, Dk)) / 2.0,
             v=g.standard_normal((B, H, T, Dv)),
             log_alpha=-g.uniform(0.05, 1.5, (B, H, T, Dk)),
             b=g.uniform(0.1, 0.9, (B, H, T, Dk)),
             w=g.uniform(0.1, 0.9, (B, H, T, Dv)),
             S0=0.5 * g.standard_normal((B, H, Dk, Dv)))
    adj = dict(do=g.standard_normal((B, H, T, Dv)),
               dS_T=g.standard_normal((B, H, Dk, Dv)))
    return x, adj


def pin_gdn2_backward(backward=None):
    """gdn2_backward_ref, every gradient element by element, against central
    differences of gdn2_ref."""
    backward = backward or BW.gdn2_backward_ref
    x, adj = _gdn2_case(9)
    scale = 0.6
    gr = backward(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"],
                  x["S0"], adj["do"], adj["dS_T"], scale)

    def loss(y):
        o, S = R.gdn2_ref(y["q"], y["k"], y["v"], y["log_alpha"], y["b"],
                          y["w"], y["S0"], scale)
        return np.sum(adj["do"] * o) + np.sum(adj["dS_T"] * S)
    names = ("q", "k", "v", "log_alpha", "b", "w", "S0")
    num = _numeric_grads(loss, x, names)
    for name in names:
        np.testing.assert_allclose(gr[name], num[name], rtol=1e-6, atol=1e-7,
                                   err_msg=name)


def test_gdn2_backward_matches_central_differences():
    pin_gdn2_backward()


def test_gdn2_backward_defaults():
    """S0 and dS_T left out equal explicit zeros."""
    x, adj = _gdn2_case(10)
    B, H, T, Dk = x["k"].shape
    Dv = x["v"].shape[-1]
    a = BW.gdn2_backward_ref(x["q"], x["k"], x["v"], x["log_alpha"], x["b"],
                             x["w"], None, adj["do"])
    z = np.zeros((B, H, Dk, Dv))
    b = BW.gdn2_backward_ref(x["q"], x["k"], x["v"], x["log_alpha"], x["b"],
                             x["w"], z, adj["do"], z)
    for n in a:
        np.testing.assert_allclose(a[n], b[n], rtol=1e-14, atol=1e-14)


def _mutant_fn(edit, fn):
    src = open(BW.__file__).read()
    assert src.count(edit[0]) == 1, edit[0]
    ns = {}
    code = src.replace(edit[0], edit[1])
    code = code.replace("from .recurrence import _f64",
                        "from oracle.recurrence import _f64")
    exec(compile(code, "mutant", "exec"), ns)
    return ns[fn]


GATED_MUTANTS = [
    # decay's gradient read off the state before the decay
    ("gla[..., t, :] = (dS_prev * S_dec).sum(-2)",
     "gla[..., t, :] = (dS_prev * S_prev).sum(-2)"),
    # decay not carried into the adjoint of S_{t-1}
    ("dS_prev = dS_prev * np.exp(la[..., t, :])[..., None, :]",
     "dS_prev = dS_prev"),
    # read key through the undecayed state
    ('dk = -bt[..., None] * np.einsum("...vk,...v->...k", S_dec, w)',
     'dk = -bt[..., None] * np.einsum("...vk,...v->...k", S_prev, w)'),
]

GDN2_MUTANTS = [
    ("dS_dec = dS - e[..., :, None] * dz[..., None, :]",
     "dS_dec = dS - kt[..., :, None] * dz[..., None, :]"),      # k for e
    ("gk[..., t, :] += bt * de", "gk[..., t, :] += 0.0 * de"),   # drop the erase path
    ("gla[..., t, :] = (dS_dec * S_dec).sum(-1)",
     "gla[..., t, :] = (dS * S_dec).sum(-1)"),                  # wrong adjoint
    ("dS = np.exp(la[..., t, :])[..., :, None] * dS_dec",
     "dS = dS_dec"),                                            # decay dropped
    ("de = -np.einsum(", "de = np.einsum("),                     # sign
    ("gw[..., t, :] = vt * dz", "gw[..., t, :] = wt * dz"),      # swapped gate
]


@pytest.mark.parametrize("edit", GATED_MUTANTS, ids=[m[1][:30] for m in GATED_MUTANTS])
def test_gated_backward_mutants_are_caught(edit):
    with pytest.raises(AssertionError):
        pin_gated_backward(_mutant_fn(edit, "osdn_gated_backward_ref"))


@pytest.mark.parametrize("edit", GDN2_MUTANTS, ids=[m[1][:30] for m in GDN2_MUTANTS])
def test_gdn2_backward_mutants_are_caught(edit):
    with pytest.raises(AssertionError):
        pin_gdn2_backward(_mutant_fn(edit, "gdn2_backward_ref"))
