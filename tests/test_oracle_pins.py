"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

None of these tests compares the oracle with itself: each checks it against a
closed form, an invariant, a special case that reduces to a textbook routine,
exact rational arithmetic with an independent unrolling, or finite
differences of a definition. ``test_mutants_are_caught`` plants plausible
mistakes in the oracle (on the CPU) and checks that some pin fails for each.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import recurrence as R
from oracle import exact as X


def _rng(seed):
    return np.random.default_rng(seed)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand_osdn(seed, B=2, H=2, T=24, Dk=6, Dv=5, apf=True):
    g = _rng(seed)
    q = _unit(g.standard_normal((B, H, T, Dk)))
    k = _unit(g.standard_normal((B, H, T, Dk)))
    v = g.standard_normal((B, H, T, Dv))
    beta = 1.0 / (1.0 + np.exp(-g.standard_normal((B, H, T))))
    r = (1.0 / (1.0 + np.exp(-g.normal(2.0, 0.5, (B, H, T))))) if apf else None
    return q, k, v, beta, r


# ---------------------------------------------------------------------------
# Pins as plain functions so the mutation test can re-run them
# ---------------------------------------------------------------------------

def pin_closed_form_equals_definition():
    """h_t by its definition (with S, v) equals the printed closed form."""
    g = _rng(1)
    for _ in range(100):
        Dk, Dv = 7, 4
        S = g.standard_normal((Dv, Dk))
        v = g.standard_normal(Dv)
        k = g.standard_normal(Dk)
        d = g.uniform(0.2, 2.0, Dk)
        beta = g.uniform(0.05, 0.95)
        hd = R.h_by_definition(S, v, d, k, beta)
        hc = R.h_closed_form(d, k, beta)
        assert abs(hd - hc) <= 1e-10 * max(1.0, abs(hc))


def pin_step_is_descent_on_definition():
    """The oracle's d-step equals -eta * (finite-difference gradient of h by
    its definition), so sign and scale follow the surrogate, not a misprint."""
    g = _rng(2)
    eta = 0.3
    for _ in range(20):
        Dk, Dv = 5, 3
        S = g.standard_normal((Dv, Dk))
        v = g.standard_normal(Dv)
        k = g.standard_normal(Dk)
        d = g.uniform(0.2, 2.0, Dk)
        beta = np.float64(g.uniform(0.05, 0.95))
        r = np.float64(g.uniform(0.5, 1.0))
        fd = np.empty(Dk)
        eps = 1e-6
        for i in range(Dk):
            e = np.zeros(Dk)
            e[i] = eps
            fd[i] = (R.h_by_definition(S, v, d + e, k, beta)
                     - R.h_by_definition(S, v, d - e, k, beta)) / (2 * eps)
        _, d_next, _, _ = R._phase1_step(d[None], k[None], beta[None],
                                         r[None], eta)
        step = d_next[0] - r * d
        np.testing.assert_allclose(step, -eta * fd, rtol=1e-6, atol=1e-9)


def pin_repeated_key_dynamics():
    """Same key, same beta, r = 1: c_t - 1/beta shrinks by (1 - m) per token,
    m = eta beta^2 ||a||^2 / n (derived from the closed form + descent)."""
    g = _rng(3)
    Dk, T, eta, beta = 8, 40, 0.7, 0.6
    k1 = _unit(g.standard_normal(Dk))
    k = np.broadcast_to(k1, (1, 1, T, Dk)).copy()
    b = np.full((1, 1, T), beta)
    d0 = g.uniform(0.5, 1.5, (1, 1, Dk))
    _, _, c, _ = R.precond_scan_ref(k, b, None, eta, d0)
    a = k1 * k1
    n = a.sum()
    m = eta * beta ** 2 * (a @ a) / n
    c1 = d0[0, 0] @ a
    expect = 1 / beta + (c1 - 1 / beta) * (1 - m) ** np.arange(T)
    np.testing.assert_allclose(c[0, 0], expect, rtol=1e-12)


def pin_constant_gate_fixed_point():
    """Same key, constant r: c converges to (eta beta |a|^2/n)/(1 - r + m)."""
    g = _rng(4)
    Dk, T, eta, beta, rr = 8, 400, 0.5, 0.7, 0.9
    k1 = _unit(g.standard_normal(Dk))
    k = np.broadcast_to(k1, (1, 1, T, Dk)).copy()
    b = np.full((1, 1, T), beta)
    r = np.full((1, 1, T), rr)
    _, _, c, _ = R.precond_scan_ref(k, b, r, eta, None)
    a = k1 * k1
    n = a.sum()
    aa = a @ a
    m = eta * beta ** 2 * aa / n
    cstar = (eta * beta * aa / n) / (1 - rr + m)
    # exact affine recursion c_{t+1} = (r - m) c_t + eta beta |a|^2 / n
    np.testing.assert_allclose(c[0, 0, 1:],
                               (rr - m) * c[0, 0, :-1] + eta * beta * aa / n,
                               rtol=1e-12)
    assert abs(c[0, 0, -1] - cstar) < 1e-12


def pin_per_token_contraction():
    """f_t(S_t) = (1 - beta_t c_t)^2 f_t(S_{t-1}) on every token (the
    residual-ratio identity behind the bounded product of Theorem 5.2)."""
    q, k, v, beta, r = _rand_osdn(5, T=30)
    o, S, d, tr, states = R.osdn_ref(q, k, v, beta, r, 0.2,
                                     return_trace=True, return_states=True)
    for t in range(k.shape[2]):
        f_new = R.regression_loss(states[t + 1], k[:, :, t], v[:, :, t])
        f_old = R.regression_loss(states[t], k[:, :, t], v[:, :, t])
        np.testing.assert_allclose(f_new, tr["rho"][:, :, t] * f_old,
                                   rtol=1e-10, atol=1e-14)


def pin_residual_ratio_is_loss_ratio():
    """residual_ratio_ref's rho_t equals the ratio of the regression losses
    f_t(S_t) / f_t(S_{t-1}) computed from the states of the full recurrence
    (random values and a random initial state), and q_geo is the T-th root
    of their product ([OSDN-it] section 3, Theorem 5.2; section 4.2)."""
    q, k, v, beta, r = _rand_osdn(15, T=40)
    g = _rng(16)
    S0 = g.standard_normal((2, 2, 5, 6))
    d0 = g.uniform(0.5, 1.5, (2, 2, 6))
    rho, qg = R.residual_ratio_ref(k, beta, r, 0.3, d0)
    _, _, _, states = R.osdn_ref(q, k, v, beta, r, 0.3, d0, S0,
                                 return_states=True)
    ratios = np.stack([R.regression_loss(states[t + 1], k[:, :, t], v[:, :, t])
                       / R.regression_loss(states[t], k[:, :, t], v[:, :, t])
                       for t in range(k.shape[2])], axis=-1)
    np.testing.assert_allclose(rho, ratios, rtol=1e-9)
    np.testing.assert_allclose(qg, np.prod(ratios, axis=-1) ** (1.0 / 40),
                               rtol=1e-9)
    # no forgetting, d0 = 1, eta = 0: plain DeltaNet, rho_t = (1 - beta_t)^2
    # for unit keys
    rho0, _ = R.residual_ratio_ref(k, beta, None, 0.0)
    np.testing.assert_allclose(rho0, (1.0 - beta) ** 2, rtol=1e-12)


def pin_gated_osdn_reductions():
    """OSDN on a decaying backbone: no decay gives OSDN exactly; d = 1, eta = 0
    and no forgetting give Kimi-style delta attention, i.e. GDN-2 with erase
    and write gates equal to beta (transposed state); and on every token the
    write contracts the loss of the DECAYED state by (1 - beta c)^2."""
    q, k, v, beta, r = _rand_osdn(21, T=25)
    g = _rng(22)
    la = -0.3 * g.random(k.shape)
    S0 = g.standard_normal((2, 2, 5, 6))
    d0 = g.uniform(0.5, 1.5, (2, 2, 6))
    o1, S1, d1 = R.osdn_gated_ref(q, k, v, beta, np.zeros(k.shape), r, 0.2,
                                  d0, S0)
    o2, S2, d2 = R.osdn_ref(q, k, v, beta, r, 0.2, d0, S0)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(S1, S2, rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(d1, d2)
    o3, S3, _ = R.osdn_gated_ref(q, k, v, beta, la, None, 0.0)
    bb = np.broadcast_to(beta[..., None], k.shape)
    ww = np.broadcast_to(beta[..., None], v.shape)
    o4, S4 = R.gdn2_ref(q, k, v, la, bb, ww)
    np.testing.assert_allclose(o3, o4, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S3, np.swapaxes(S4, -1, -2), rtol=1e-11,
                               atol=1e-12)
    _, _, _, states = R.osdn_gated_ref(q, k, v, beta, la, r, 0.2, d0, S0,
                                       return_states=True)
    _, _, c, _ = R.precond_scan_ref(k, beta, r, 0.2, d0)
    for t in range(k.shape[2]):
        dec = states[t] * np.exp(la[:, :, t])[:, :, None, :]
        f_new = R.regression_loss(states[t + 1], k[:, :, t], v[:, :, t])
        f_old = R.regression_loss(dec, k[:, :, t], v[:, :, t])
        np.testing.assert_allclose(f_new, (1 - beta[:, :, t] * c[:, :, t]) ** 2
                                   * f_old, rtol=1e-10, atol=1e-14)


def pin_exact_unrolled():
    """fp64 oracle vs exact rationals vs the transition-product unrolling."""
    g = _rng(6)
    T, Dk, Dv = 5, 3, 2

    def rat(x, den=8):
        return [[Fraction(int(round(e * den)), den) for e in row] for row in x]

    k = rat(g.standard_normal((T, Dk)))
    q = rat(g.standard_normal((T, Dk)))
    v = rat(g.standard_normal((T, Dv)))
    beta = [Fraction(int(g.integers(1, 8)), 8) for _ in range(T)]
    r = [Fraction(int(g.integers(5, 9)), 8) for _ in range(T)]
    d0 = [Fraction(int(g.integers(4, 12)), 8) for _ in range(Dk)]
    S0 = rat(g.standard_normal((Dv, Dk)))
    eta = Fraction(1, 4)
    o_x, S_x, d_x, ktil, states = X.osdn_exact(q, k, v, beta, r, eta, d0, S0)
    S_u = X.osdn_unrolled_state(k, v, beta, ktil, S0)
    d_u, ds = X.precond_unrolled(k, beta, r, eta, d0)
    assert S_u == S_x
    assert d_u == d_x
    assert ktil == [[di * ki for di, ki in zip(ds[t], k[t])] for t in range(T)]
    f = lambda a: np.array(a, dtype=np.float64)
    o, S, d = R.osdn_ref(f(q)[None, None], f(k)[None, None], f(v)[None, None],
                         f(beta)[None, None], f(r)[None, None], float(eta),
                         f(d0)[None, None], f(S0)[None, None])
    np.testing.assert_allclose(S[0, 0], f(S_u), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(d[0, 0], f(d_u), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(o[0, 0], f(o_x), rtol=1e-12, atol=1e-13)


def pin_deltanet_reduction():
    """d = 1, eta = 0, r = 1: OSDN is plain DeltaNet, and DeltaNet's state is
    the transition-product unrolling with k~ = k."""
    q, k, v, beta, _ = _rand_osdn(7, T=20)
    o, S, d = R.osdn_ref(q, k, v, beta, None, 0.0, None, None)
    o2, S2 = R.deltanet_ref(q, k, v, beta)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(S, S2, rtol=0, atol=1e-14)
    assert np.all(d == 1.0)
    # unrolled product, one (b, h), in fp64 with Fractions of the same floats
    kk = [[Fraction(e) for e in row] for row in k[0, 0]]
    vv = [[Fraction(e) for e in row] for row in v[0, 0, :8]]
    S_u = X.osdn_unrolled_state(kk[:8], vv, [Fraction(b) for b in beta[0, 0, :8]],
                                kk[:8], [[0] * k.shape[-1]] * v.shape[-1])
    _, S8 = R.deltanet_ref(q[:, :, :8], k[:, :, :8], v[:, :, :8], beta[:, :, :8])
    np.testing.assert_allclose(S8[0, 0], np.array(S_u, dtype=np.float64),
                               rtol=1e-12, atol=1e-14)


def pin_newton_condition():
    """beta <d, k^2> = 1 (gated Newton condition): the write is exact,
    S_1 k_1 = v_1, the surrogate is at its minimum -1/(2n) and the step is 0."""
    k = [[Fraction(1, 2), Fraction(-1, 4), Fraction(3, 4)]]
    q = [[Fraction(1), Fraction(0), Fraction(0)]]
    v = [[Fraction(5, 3), Fraction(-2, 7)]]
    beta = [Fraction(2, 5)]
    n = sum(x * x for x in k[0])
    d0 = [1 / (beta[0] * n)] * 3
    S0 = [[Fraction(1, 3), 0, Fraction(-1, 2)], [Fraction(2), Fraction(1, 5), 0]]
    o, S, d, ktil, states = X.osdn_exact(q, k, v, beta, [Fraction(9, 10)],
                                        Fraction(1, 3), d0, S0)
    Sk = [sum(S[i][j] * k[0][j] for j in range(3)) for i in range(2)]
    assert Sk == v[0]
    assert d == [Fraction(9, 10) * x for x in d0]   # g_1 = 0
    hc = R.h_closed_form(np.array(d0, float), np.array(k[0], float),
                         float(beta[0]))
    assert abs(hc + 1 / (2 * float(n))) < 1e-15
    gr = R.grad_h_closed_form(np.array(d0, float), np.array(k[0], float),
                              float(beta[0]))
    assert np.all(np.abs(gr) < 1e-15)


def pin_degenerate_gates():
    """beta = 0: memory untouched, o_t = S_0 q_t, d_{t+1} = r_t d_t.
    eta = 0: d_t = (prod of r) d_0."""
    q, k, v, beta, r = _rand_osdn(8, T=15)
    g = _rng(8)
    S0 = g.standard_normal((2, 2, v.shape[-1], k.shape[-1]))
    d0 = g.uniform(0.5, 2, (2, 2, k.shape[-1]))
    o, S, d = R.osdn_ref(q, k, v, np.zeros_like(beta), r, 0.3, d0, S0)
    np.testing.assert_array_equal(S, S0)
    np.testing.assert_allclose(o, np.einsum("bhvk,bhtk->bhtv", S0, q),
                               rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(d, d0 * np.prod(r, axis=-1)[..., None],
                               rtol=1e-13)
    kt, d2, _, _ = R.precond_scan_ref(k, beta, r, 0.0, d0)
    cum = np.concatenate([np.ones((2, 2, 1)), np.cumprod(r, axis=-1)[..., :-1]],
                         axis=-1)
    np.testing.assert_allclose(kt, cum[..., None] * d0[:, :, None, :] * k,
                               rtol=1e-13)


def pin_readout_inclusive():
    """o_t = S_t q_t with S_t the state after token t."""
    q, k, v, beta, r = _rand_osdn(9, T=12)
    o, S, d, states = R.osdn_ref(q, k, v, beta, r, 0.1, return_states=True)
    for t in range(12):
        np.testing.assert_allclose(
            o[:, :, t], np.einsum("bhvk,bhk->bhv", states[t + 1], q[:, :, t]),
            rtol=1e-13, atol=1e-14)


def pin_gdn2_exact_and_orientation():
    """GDN-2: fp64 vs exact vs the transition-product unrolling; exact erase
    when k^T(b*k) = 1 (the read S^T e_t becomes z_t)."""
    g = _rng(10)
    T, Dk, Dv = 4, 3, 2

    def rat(x, den=8):
        return [[Fraction(int(round(e * den)), den) for e in row] for row in x]

    k = rat(g.standard_normal((T, Dk)))
    q = rat(g.standard_normal((T, Dk)))
    v = rat(g.standard_normal((T, Dv)))
    alpha = [[Fraction(int(g.integers(4, 9)), 8) for _ in range(Dk)]
             for _ in range(T)]
    b = [[Fraction(int(g.integers(0, 9)), 8) for _ in range(Dk)]
         for _ in range(T)]
    w = [[Fraction(int(g.integers(0, 9)), 8) for _ in range(Dv)]
         for _ in range(T)]
    S0 = rat(g.standard_normal((Dk, Dv)))
    o_x, S_x, _ = X.gdn2_exact(q, k, v, alpha, b, w, S0)
    assert X.gdn2_unrolled_state(k, v, alpha, b, w, S0) == S_x
    f = lambda a: np.array(a, dtype=np.float64)[None, None]
    o, S = R.gdn2_ref(f(q), f(k), f(v), np.log(f(alpha)), f(b), f(w),
                      f(S0)[0])
    np.testing.assert_allclose(S[0, 0], f(S_x)[0, 0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(o[0, 0], f(o_x)[0, 0], rtol=1e-12, atol=1e-13)
    # exact erase: k = (1, 1, 0), b = (1/2, 1/2, 1) => k^T (b*k) = 1
    k1 = [[1, 1, 0]]
    b1 = [[Fraction(1, 2), Fraction(1, 2), 1]]
    w1 = [[1, Fraction(1, 3)]]
    v1 = [[Fraction(3), Fraction(-6)]]
    _, S1, _ = X.gdn2_exact([[0, 0, 0]], k1, v1, [[1, 1, 1]], b1, w1, S0)
    e = [Fraction(1, 2), Fraction(1, 2), 0]
    read = [sum(S1[i][j] * e[i] for i in range(3)) for j in range(2)]
    assert read == [Fraction(3), Fraction(-2)]


def pin_gdn2_reductions():
    """b = w = beta, alpha = 1: GDN-2 is DeltaNet with the state transposed."""
    q, k, v, beta, _ = _rand_osdn(11, T=16)
    Dk, Dv = k.shape[-1], v.shape[-1]
    bb = np.broadcast_to(beta[..., None], k.shape)
    ww = np.broadcast_to(beta[..., None], v.shape)
    o, S = R.gdn2_ref(q, k, v, np.zeros(k.shape), bb, ww)
    o2, S2 = R.deltanet_ref(q, k, v, beta)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S, np.swapaxes(S2, -1, -2), rtol=1e-12,
                               atol=1e-13)


def pin_grad_h_scale():
    """grad_h_closed_form equals the central-difference gradient of h, taken
    both from the printed closed form and from h's definition with a random
    state and value ([OSDN-it] section 2.2), in direction and in scale
    (keys of random norm, so a dropped 1/||k||^2 or beta shows)."""
    g = _rng(23)
    eps = 1e-6
    for _ in range(25):
        Dk, Dv = 6, 4
        k = g.standard_normal(Dk) * g.uniform(0.3, 3.0)
        d = g.uniform(0.2, 2.0, Dk)
        beta = g.uniform(0.05, 0.95)
        S = g.standard_normal((Dv, Dk))
        v = g.standard_normal(Dv)
        fd_c = np.empty(Dk)
        fd_d = np.empty(Dk)
        for i in range(Dk):
            e = np.zeros(Dk)
            e[i] = eps
            fd_c[i] = (R.h_closed_form(d + e, k, beta)
                       - R.h_closed_form(d - e, k, beta)) / (2 * eps)
            fd_d[i] = (R.h_by_definition(S, v, d + e, k, beta)
                       - R.h_by_definition(S, v, d - e, k, beta)) / (2 * eps)
        gr = R.grad_h_closed_form(d, k, beta)
        np.testing.assert_allclose(gr, fd_c, rtol=1e-6, atol=1e-10)
        np.testing.assert_allclose(gr, fd_d, rtol=1e-6, atol=1e-10)


PINS = [
    pin_closed_form_equals_definition,
    pin_step_is_descent_on_definition,
    pin_repeated_key_dynamics,
    pin_constant_gate_fixed_point,
    pin_per_token_contraction,
    pin_residual_ratio_is_loss_ratio,
    pin_gated_osdn_reductions,
    pin_exact_unrolled,
    pin_deltanet_reduction,
    pin_newton_condition,
    pin_degenerate_gates,
    pin_readout_inclusive,
    pin_gdn2_exact_and_orientation,
    pin_gdn2_reductions,
    pin_grad_h_scale,
]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ---------------------------------------------------------------------------
# Further properties
# ---------------------------------------------------------------------------

def test_closed_form_independent_of_state_and_value():
    g = _rng(12)
    d = g.uniform(0.3, 1.7, 6)
    k = g.standard_normal(6)
    hs = [R.h_by_definition(g.standard_normal((4, 6)), g.standard_normal(4),
                            d, k, 0.35) for _ in range(20)]
    assert np.ptp(hs) < 1e-12


def test_descent_lowers_surrogate_and_ascent_raises_it():
    g = _rng(13)
    for _ in range(20):
        k = g.standard_normal(6)
        d = g.uniform(0.1, 3.0, 6)
        beta = g.uniform(0.1, 0.9)
        grad = R.grad_h_closed_form(d, k, beta)
        if np.linalg.norm(grad) < 1e-9:
            continue
        eta = 1e-3
        h0 = R.h_closed_form(d, k, beta)
        assert R.h_closed_form(d - eta * grad, k, beta) < h0
        assert R.h_closed_form(d + eta * grad, k, beta) > h0


def test_ascent_reading_diverges_on_repeated_key():
    """The printed '+' sign would push c_t away from 1/beta geometrically."""
    g = _rng(14)
    Dk, T, eta, beta = 8, 60, 0.7, 0.6
    k1 = _unit(g.standard_normal(Dk))
    a = k1 * k1
    n = a.sum()
    d = np.full(Dk, 0.5)
    devs = []
    for _ in range(T):
        c = d @ a
        devs.append(abs(c - 1 / beta))
        d = d - eta * beta * (1 - beta * c) / n * a     # ascent
    assert devs[-1] > 2 * devs[0]


def test_decoupling_phase1_reads_only_keys():
    q, k, v, beta, r = _rand_osdn(15, T=18)
    g = _rng(15)
    _, _, d1, tr1 = R.osdn_ref(q, k, v, beta, r, 0.2, return_trace=True)
    _, _, d2, tr2 = R.osdn_ref(g.standard_normal(q.shape), k,
                               g.standard_normal(v.shape), beta, r, 0.2,
                               S0=g.standard_normal((2, 2, 5, 6)),
                               return_trace=True)
    np.testing.assert_array_equal(d1, d2)
    np.testing.assert_array_equal(tr1["ktilde"], tr2["ktilde"])
    kt, d3, _, _ = R.precond_scan_ref(k, beta, r, 0.2)
    np.testing.assert_array_equal(kt, tr1["ktilde"])
    np.testing.assert_array_equal(d3, d1)


def test_state_carry():
    q, k, v, beta, r = _rand_osdn(16, T=30)
    o, S, d = R.osdn_ref(q, k, v, beta, r, 0.2)
    s = 13
    oa, Sa, da = R.osdn_ref(q[:, :, :s], k[:, :, :s], v[:, :, :s],
                            beta[:, :, :s], r[:, :, :s], 0.2)
    ob, Sb, db = R.osdn_ref(q[:, :, s:], k[:, :, s:], v[:, :, s:],
                            beta[:, :, s:], r[:, :, s:], 0.2, da, Sa)
    np.testing.assert_allclose(np.concatenate([oa, ob], axis=2), o, rtol=1e-13,
                               atol=1e-14)
    np.testing.assert_allclose(Sb, S, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(db, d, rtol=1e-13)


def test_zero_key_is_a_no_op_for_the_step():
    q, k, v, beta, r = _rand_osdn(17, T=8)
    k[:, :, 3] = 0.0
    _, _, c, gg = R.precond_scan_ref(k, beta, r, 0.2)
    assert np.all(gg[:, :, 3] == 0.0)
    o, S, d = R.osdn_ref(q, k, v, beta, r, 0.2)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(d))


# ---------------------------------------------------------------------------
# Mutation check: plant mistakes in the oracle, on the CPU
# ---------------------------------------------------------------------------

def _mut_ascent(d, kt, beta_t, r_t, eta):
    kt_, dn, c, g = _ORIG_STEP(d, kt, beta_t, r_t, eta)
    a = kt * kt
    return kt_, r_t[..., None] * d - g[..., None] * a, c, -g


def _mut_grad_at_gated(d, kt, beta_t, r_t, eta):
    return _ORIG_STEP(r_t[..., None] * d, kt, beta_t, np.ones_like(r_t), eta)


def _mut_ktilde_after_update(d, kt, beta_t, r_t, eta):
    kt_, dn, c, g = _ORIG_STEP(d, kt, beta_t, r_t, eta)
    return dn * kt, dn, c, g


def _mut_norm_not_squared(d, kt, beta_t, r_t, eta):
    kt_, dn, c, g = _ORIG_STEP(d, kt, beta_t, r_t, eta)
    n = np.sum(kt * kt, axis=-1)
    g2 = g * n / np.sqrt(n)
    return kt_, r_t[..., None] * d + g2[..., None] * (kt * kt), c, g2


def _mut_plain_key_dot(d, kt, beta_t, r_t, eta):
    # c_t = <d, k> instead of <d, k*k>
    a = kt * kt
    n = np.sum(a, axis=-1)
    c = np.sum(d * kt, axis=-1)
    g = eta * beta_t * (1.0 - beta_t * c) / n
    return d * kt, r_t[..., None] * d + g[..., None] * a, c, g


_ORIG_STEP = R._phase1_step
_ORIG_GRAD = R.grad_h_closed_form


def _mut_grad_no_norm(d, k, beta):
    # the 1 / ||k||^2 factor dropped
    n = np.sum(np.asarray(k, float) ** 2, axis=-1)
    return _ORIG_GRAD(d, k, beta) * np.asarray(n)[..., None]


def _mut_grad_one_beta(d, k, beta):
    # one factor beta dropped: -(1 - beta c) a / n
    return _ORIG_GRAD(d, k, beta) / np.asarray(beta, float)[..., None]


def _mut_grad_sign(d, k, beta):
    return -_ORIG_GRAD(d, k, beta)


MUTANTS = [("_phase1_step", m) for m in (_mut_ascent, _mut_grad_at_gated,
                                         _mut_ktilde_after_update,
                                         _mut_norm_not_squared,
                                         _mut_plain_key_dot)]
MUTANTS += [("grad_h_closed_form", m) for m in (_mut_grad_no_norm,
                                                _mut_grad_one_beta,
                                                _mut_grad_sign)]


@pytest.mark.parametrize("attr,mutant", MUTANTS,
                         ids=[m.__name__ for _, m in MUTANTS])
def test_mutants_are_caught(monkeypatch, attr, mutant):
    monkeypatch.setattr(R, attr, mutant)
    failed = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "no pin caught mutant %s" % mutant.__name__
