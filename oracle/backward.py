"""fp64 reverse-mode adjoint of the OSDN token recurrence (the backward pass).

TEST INFRASTRUCTURE ONLY: imported by the tests and the benchmark's CPU
baseline, never by the HIP library.

The forward is osdn_ref in recurrence.py ([OSDN-it] sections 2.1-2.3): per
(batch, head) and token t,

    a = k_t*k_t, n = ||k_t||^2, c = <d_t, a>, k~ = d_t*k_t
    u = v_t - S_{t-1} k_t
    S_t = S_{t-1} + beta_t u k~^T
    o_t = scale * S_t q_t
    g = eta beta_t (1 - beta_t c) / n        (0 when n = 0)
    d_{t+1} = r_t d_t + g a.

Given the adjoints of the outputs (do, dS_T, dd_T) this returns the adjoints
of every input, i.e. the gradient of L = <do, o> + <dS_T, S_T> + <dd_T, d_T>.
It walks the tokens backwards, applying the chain rule to the lines above in
reverse order; the states S_{t-1} are those the forward stored. Nothing here
is blocked or reordered: it is the plain adjoint of the plain recurrence,
checked against central differences of osdn_ref in the tests.

Readings: the zero-key convention of the forward (g = 0 when n = 0) carries
over, so no gradient flows through g at such a token; eta is a scalar shared
by all (batch, head) streams, and its adjoint is returned per stream
([B, H]); a caller sums it.
"""

import numpy as np

from .recurrence import _f64


def osdn_backward_ref(q, k, v, beta, r, eta, d0, S0, do, dS_T=None, dd_T=None,
                      scale=1.0):
    """Adjoint of osdn_ref. Shapes as in osdn_ref; do [B,H,T,Dv], dS_T
    [B,H,Dv,Dk] and dd_T [B,H,Dk] (None: zero). r, d0, S0 as in osdn_ref
    (None: ones, ones, zeros).

    Returns dict(q, k, v, beta, r, eta, d0, S0) of fp64 gradients; r's
    gradient is there even when r is None (the gradient at r = 1), eta's is
    per (batch, head) [B, H].
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    lead = k.shape[:-2]
    T, Dk = k.shape[-2], k.shape[-1]
    Dv = v.shape[-1]
    r = np.ones(beta.shape) if r is None else _f64(r)
    d = np.ones(lead + (Dk,)) if d0 is None else np.array(d0, dtype=np.float64)
    S = (np.zeros(lead + (Dv, Dk)) if S0 is None
         else np.array(S0, dtype=np.float64))
    do = _f64(do)

    # forward, keeping what the adjoint needs
    Sprev, ds, us, gs, cs, ns = [], [], [], [], [], []
    for t in range(T):
        kt = k[..., t, :]
        a = kt * kt
        n = a.sum(-1)
        c = (d * a).sum(-1)
        kt_ = d * kt
        u = v[..., t, :] - np.einsum("...vk,...k->...v", S, kt)
        Sprev.append(S)
        ds.append(d)
        us.append(u)
        cs.append(c)
        ns.append(n)
        S = S + beta[..., t, None, None] * u[..., :, None] * kt_[..., None, :]
        safe_n = np.where(n > 0.0, n, 1.0)
        g = np.where(n > 0.0, eta * beta[..., t] * (1.0 - beta[..., t] * c) / safe_n,
                     0.0)
        gs.append(g)
        d = r[..., t, None] * d + g[..., None] * a

    # reverse
    dS = np.zeros(lead + (Dv, Dk)) if dS_T is None else np.array(dS_T, np.float64)
    dd = np.zeros(lead + (Dk,)) if dd_T is None else np.array(dd_T, np.float64)
    gq, gk, gv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    gb, gr = np.zeros(beta.shape), np.zeros(beta.shape)
    geta = np.zeros(lead)
    S_after = S
    for t in reversed(range(T)):
        kt, qt, bt, rt = k[..., t, :], q[..., t, :], beta[..., t], r[..., t]
        d_t, u, g, c, n = ds[t], us[t], gs[t], cs[t], ns[t]
        a = kt * kt
        kt_ = d_t * kt
        S_prev = Sprev[t]
        # o_t = scale S_t q_t
        dS = dS + scale * do[..., t, :, None] * qt[..., None, :]
        gq[..., t, :] = scale * np.einsum("...vk,...v->...k", S_after, do[..., t, :])
        # S_t = S_{t-1} + beta u k~^T, u = v - S_{t-1} k
        w = np.einsum("...vk,...k->...v", dS, kt_)
        gv[..., t, :] = bt[..., None] * w
        gb[..., t] = (u * w).sum(-1)
        dkt_ = bt[..., None] * np.einsum("...vk,...v->...k", dS, u)
        dk = -bt[..., None] * np.einsum("...vk,...v->...k", S_prev, w)
        dS_prev = dS - bt[..., None, None] * w[..., :, None] * kt[..., None, :]
        # k~ = d_t * k_t
        dd_t = dkt_ * kt
        dk = dk + dkt_ * d_t
        # d_{t+1} = r d_t + g a  (dd is the adjoint of d_{t+1})
        gr[..., t] = (dd * d_t).sum(-1)
        dg = (dd * a).sum(-1)
        da = g[..., None] * dd
        dd_t = dd_t + rt[..., None] * dd
        # g = eta beta (1 - beta c) / n, only where n > 0
        safe_n = np.where(n > 0.0, n, 1.0)
        live = n > 0.0
        dc = np.where(live, -eta * bt * bt / safe_n * dg, 0.0)
        gb[..., t] += np.where(live, eta * (1.0 - 2.0 * bt * c) / safe_n * dg, 0.0)
        dn = np.where(live, -g / safe_n * dg, 0.0)
        geta += np.where(live, bt * (1.0 - bt * c) / safe_n * dg, 0.0)
        # c = <d_t, a>, n = sum a, a = k*k
        dd_t = dd_t + dc[..., None] * a
        da = da + dc[..., None] * d_t + dn[..., None]
        dk = dk + 2.0 * kt * da
        gk[..., t, :] = dk
        dd = dd_t
        dS = dS_prev
        S_after = S_prev
    return dict(q=gq, k=gk, v=gv, beta=gb, r=gr, eta=geta, d0=dd, S0=dS)
