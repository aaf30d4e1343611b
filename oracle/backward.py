"""fp64 reverse-mode adjoints of the token recurrences (the backward pass).

TEST INFRASTRUCTURE ONLY: imported by the tests and the benchmark's CPU
baseline, never by the HIP library.

osdn_backward_ref is the adjoint of osdn_ref ([OSDN-it] sections 2.1-2.3):
per (batch, head) and token t,

    a = k_t*k_t, n = ||k_t||^2, c = <d_t, a>, k~ = d_t*k_t
    u = v_t - S_{t-1} k_t
    S_t = S_{t-1} + beta_t u k~^T
    o_t = scale * S_t q_t
    g = eta beta_t (1 - beta_t c) / n        (0 when n = 0)
    d_{t+1} = r_t d_t + g a.

osdn_gated_backward_ref is the adjoint of osdn_gated_ref (the same step on a
per-key-channel-decay backbone: S_{t-1} is first replaced by
S_{t-1} Diag(alpha_t)), and gdn2_backward_ref that of gdn2_ref ([GDN2-it]
method, part 1: decay, erase gate and write gate; state [Dk, Dv]).

Given the adjoints of the outputs (do, dS_T, and dd_T for OSDN) each returns
the adjoints of every input, i.e. the gradient of
L = <do, o> + <dS_T, S_T> (+ <dd_T, d_T>). It walks the tokens backwards,
applying the chain rule to the lines of the forward in reverse order; the
states the forward passed through are those it stored. Nothing here is
blocked or reordered: it is the plain adjoint of the plain recurrence,
checked against central differences of the forward oracles in the tests.

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
    return _osdn_adjoint(q, k, v, beta, None, r, eta, d0, S0, do, dS_T, dd_T,
                         scale)


def osdn_gated_backward_ref(q, k, v, beta, log_alpha, r, eta, d0, S0, do,
                            dS_T=None, dd_T=None, scale=1.0):
    """Adjoint of osdn_gated_ref: as osdn_backward_ref, with the per-channel
    decay log_alpha [B,H,T,Dk]; the result also holds log_alpha's gradient.
    With S_dec = S_{t-1} Diag(alpha_t) the step reads and writes S_dec, so
    the adjoint of S_dec is that of S_t less the write's, and
    dL/dlog alpha_t[j] = sum_i dS_dec[i, j] S_dec[i, j],
    dS_{t-1} = dS_dec Diag(alpha_t)."""
    return _osdn_adjoint(q, k, v, beta, log_alpha, r, eta, d0, S0, do, dS_T,
                         dd_T, scale)


def _osdn_adjoint(q, k, v, beta, log_alpha, r, eta, d0, S0, do, dS_T, dd_T,
                  scale):
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    lead = k.shape[:-2]
    T, Dk = k.shape[-2], k.shape[-1]
    Dv = v.shape[-1]
    r = np.ones(beta.shape) if r is None else _f64(r)
    d = np.ones(lead + (Dk,)) if d0 is None else np.array(d0, dtype=np.float64)
    S = (np.zeros(lead + (Dv, Dk)) if S0 is None
         else np.array(S0, dtype=np.float64))
    do = _f64(do)
    la = None if log_alpha is None else _f64(log_alpha)

    # forward, keeping what the adjoint needs
    Sprev, Sdec, ds, us, gs, cs, ns = [], [], [], [], [], [], []
    for t in range(T):
        kt = k[..., t, :]
        a = kt * kt
        n = a.sum(-1)
        c = (d * a).sum(-1)
        kt_ = d * kt
        Sprev.append(S)
        if la is not None:
            S = S * np.exp(la[..., t, :])[..., None, :]
        Sdec.append(S)
        u = v[..., t, :] - np.einsum("...vk,...k->...v", S, kt)
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
    gla = None if la is None else np.zeros_like(la)
    S_after = S
    for t in reversed(range(T)):
        kt, qt, bt, rt = k[..., t, :], q[..., t, :], beta[..., t], r[..., t]
        d_t, u, g, c, n = ds[t], us[t], gs[t], cs[t], ns[t]
        a = kt * kt
        kt_ = d_t * kt
        S_prev, S_dec = Sprev[t], Sdec[t]
        # o_t = scale S_t q_t
        dS = dS + scale * do[..., t, :, None] * qt[..., None, :]
        gq[..., t, :] = scale * np.einsum("...vk,...v->...k", S_after, do[..., t, :])
        # S_t = S_dec + beta u k~^T, u = v - S_dec k (S_dec = S_{t-1}
        # without decay)
        w = np.einsum("...vk,...k->...v", dS, kt_)
        gv[..., t, :] = bt[..., None] * w
        gb[..., t] = (u * w).sum(-1)
        dkt_ = bt[..., None] * np.einsum("...vk,...v->...k", dS, u)
        dk = -bt[..., None] * np.einsum("...vk,...v->...k", S_dec, w)
        dS_prev = dS - bt[..., None, None] * w[..., :, None] * kt[..., None, :]
        # S_dec = S_{t-1} Diag(exp(log alpha_t))
        if la is not None:
            gla[..., t, :] = (dS_prev * S_dec).sum(-2)
            dS_prev = dS_prev * np.exp(la[..., t, :])[..., None, :]
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
    out = dict(q=gq, k=gk, v=gv, beta=gb, r=gr, eta=geta, d0=dd, S0=dS)
    if la is not None:
        out["log_alpha"] = gla
    return out


def gdn2_backward_ref(q, k, v, log_alpha, b, w, S0, do, dS_T=None, scale=1.0):
    """Adjoint of gdn2_ref ([GDN2-it] method, part 1). Per token, with
    e = b*k, z = w*v and state S [Dk, Dv]:
      S_dec = Diag(alpha_t) S_{t-1}, read = S_dec^T e,
      S_t = S_dec + k (z - read)^T,  o_t = scale * S_t^T q_t.
    Shapes as in gdn2_ref; do [B,H,T,Dv], dS_T [B,H,Dk,Dv] (None: zero),
    S0 None: zeros. Returns dict(q, k, v, log_alpha, b, w, S0) of fp64
    gradients."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    la, b, w = _f64(log_alpha), _f64(b), _f64(w)
    lead = k.shape[:-2]
    T, Dk = k.shape[-2], k.shape[-1]
    Dv = v.shape[-1]
    S = (np.zeros(lead + (Dk, Dv)) if S0 is None
         else np.array(S0, dtype=np.float64))
    do = _f64(do)

    # forward, keeping each token's entry state, decayed state and read
    Sprev, Sdec, reads = [], [], []
    for t in range(T):
        Sprev.append(S)
        S = np.exp(la[..., t, :])[..., :, None] * S
        e = b[..., t, :] * k[..., t, :]
        read = np.einsum("...kv,...k->...v", S, e)
        Sdec.append(S)
        reads.append(read)
        z = w[..., t, :] * v[..., t, :]
        S = S + k[..., t, :, None] * (z - read)[..., None, :]

    # reverse
    dS = np.zeros(lead + (Dk, Dv)) if dS_T is None else np.array(dS_T, np.float64)
    gq, gk, gv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    gla, gb, gw = np.zeros_like(la), np.zeros_like(b), np.zeros_like(w)
    S_after = S
    for t in reversed(range(T)):
        kt, qt, bt, wt, vt = (k[..., t, :], q[..., t, :], b[..., t, :],
                              w[..., t, :], v[..., t, :])
        S_dec, read = Sdec[t], reads[t]
        e, z = bt * kt, wt * vt
        # o_t = scale S_t^T q_t
        dS = dS + scale * qt[..., :, None] * do[..., t, None, :]
        gq[..., t, :] = scale * np.einsum("...kv,...v->...k", S_after,
                                          do[..., t, :])
        # S_t = S_dec + k (z - read)^T
        dz = np.einsum("...kv,...k->...v", dS, kt)
        gk[..., t, :] = np.einsum("...kv,...v->...k", dS, z - read)
        gw[..., t, :] = vt * dz
        gv[..., t, :] = wt * dz
        # read = S_dec^T e: its adjoint is -dz
        de = -np.einsum("...kv,...v->...k", S_dec, dz)
        dS_dec = dS - e[..., :, None] * dz[..., None, :]
        gk[..., t, :] += bt * de
        gb[..., t, :] = kt * de
        # S_dec = Diag(exp(log alpha_t)) S_{t-1}
        gla[..., t, :] = (dS_dec * S_dec).sum(-1)
        dS = np.exp(la[..., t, :])[..., :, None] * dS_dec
        S_after = Sprev[t]
    return dict(q=gq, k=gk, v=gv, log_alpha=gla, b=gb, w=gw, S0=dS)
