"""fp64 token-by-token oracle for the OSDN forward pass and for GDN-2.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark, never by the HIP library.

Everything here is the plain recurrence the pages define, one token at a time,
in float64, vectorised only over the independent leading (batch, head) axes.
There is no chunking, blocking, fusion or reordering. The chunked WY form the
GPU uses is an exact algebraic rewrite of this recurrence; this file is the
definition it is checked against.

Layout (all arrays are NumPy, any float dtype, widened to float64 exactly):

* q, k: [B, H, T, Dk]; v: [B, H, T, Dv]; beta, r: [B, H, T]
* OSDN state S: [B, H, Dv, Dk] (so that the read is S @ k_t); d: [B, H, Dk]
* GDN-2 state S: [B, H, Dk, Dv] (the read is S^T @ e_t, the output S^T @ q_t)

Readings of points the pages leave open:

* Preconditioner step sign: descent, d_{t+1} = r_t d_t - eta * grad h_t(d_t).
  [OSDN-it] section 2.3 prints a plus sign in front of the gradient, while
  section 2.2 says d is updated by online gradient DESCENT; the descent sign
  is used.
* The gradient is taken at d_t (the value used for the write), and r_t scales
  d_t only. There is no projection or clipping of d.
* k~_t = d_t * k_t uses d_t before its update; d0 is d_1; the returned d_T is
  the preconditioner after the last token (d_{T+1}).
* Readout: o_t = scale * S_t q_t, taken after the token-t update (inclusive).
  scale = 1 is the plain reading.
* Zero key (||k_t|| = 0): h_t is undefined; the step g_t is taken as 0.
* k_t^2 inside <d_t, k_t^2> is the element-wise square.
"""

import numpy as np


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# The inner objective and the hypergradient surrogate
# ---------------------------------------------------------------------------

def regression_loss(S, k, v):
    """Per-token regression loss f_t(S) = 1/2 ||S k_t - v_t||^2.

    [OSDN-it] section 1 (problem statement): the delta rule is one online
    gradient step on this loss. S: [..., Dv, Dk], k: [..., Dk], v: [..., Dv].
    """
    S, k, v = _f64(S), _f64(k), _f64(v)
    res = np.einsum("...vk,...k->...v", S, k) - v
    return 0.5 * np.sum(res * res, axis=-1)


def osdn_write(S_prev, v, d, k, beta):
    """One OSDN memory update, S_t = S_{t-1} + beta (v - S_{t-1} k)(d * k)^T.

    [OSDN-it] section 2.1: right-preconditioning the gradient step with
    diag(d) is the same as scaling the write-side key by d.
    """
    S_prev, v, d, k = _f64(S_prev), _f64(v), _f64(d), _f64(k)
    beta = _f64(beta)
    u = v - np.einsum("...vk,...k->...v", S_prev, k)
    kt = d * k
    return S_prev + beta[..., None, None] * u[..., :, None] * kt[..., None, :]


def h_by_definition(S_prev, v, d, k, beta):
    """Surrogate h_t(d) evaluated from its definition, with the state.

    [OSDN-it] section 2.2: h_t(d) is the change of f_t produced by the
    preconditioned write, divided by the squared Frobenius norm of the
    gradient of f_t at S_{t-1}. The gradient of f_t at S is (S k - v) k^T, so
    its squared norm is ||S k - v||^2 ||k||^2.
    """
    S_prev, v, d, k = _f64(S_prev), _f64(v), _f64(d), _f64(k)
    S_new = osdn_write(S_prev, v, d, k, beta)
    res = np.einsum("...vk,...k->...v", S_prev, k) - v
    grad = res[..., :, None] * k[..., None, :]
    gnorm2 = np.sum(grad * grad, axis=(-2, -1))
    return (regression_loss(S_new, k, v) - regression_loss(S_prev, k, v)) / gnorm2


def h_closed_form(d, k, beta):
    """Closed form of the surrogate, free of S, v and the residual.

    [OSDN-it] section 2.2: h_t(d) = ((1 - beta <d, k*k>)^2 - 1) / (2 ||k||^2).
    """
    d, k, beta = _f64(d), _f64(k), _f64(beta)
    a = k * k
    c = np.sum(d * a, axis=-1)
    n = np.sum(a, axis=-1)
    return ((1.0 - beta * c) ** 2 - 1.0) / (2.0 * n)


def grad_h_closed_form(d, k, beta):
    """Gradient of the closed-form surrogate with respect to d.

    Differentiating the [OSDN-it] section 2.2 closed form:
    grad_d h_t(d) = -beta (1 - beta <d, a>) a / ||k||^2, with a = k * k.
    """
    d, k, beta = _f64(d), _f64(k), _f64(beta)
    a = k * k
    c = np.sum(d * a, axis=-1)
    n = np.sum(a, axis=-1)
    return (-beta * (1.0 - beta * c) / n)[..., None] * a


# ---------------------------------------------------------------------------
# Phase 1: the preconditioner scan (depends on k, beta, r, eta, d0 only)
# ---------------------------------------------------------------------------

def _phase1_step(d, kt, beta_t, r_t, eta):
    """One token of the preconditioner learner.

    Returns (k~_t, d_{t+1}, c_t, g_t) where c_t = <d_t, k_t*k_t> and
    d_{t+1} = r_t d_t + g_t (k_t*k_t), g_t = eta beta_t (1 - beta_t c_t)/||k_t||^2,
    which is r_t d_t - eta * grad h_t(d_t) ([OSDN-it] sections 2.2 and 2.3,
    descent sign).
    """
    a = kt * kt
    n = np.sum(a, axis=-1)
    c = np.sum(d * a, axis=-1)
    ktil = d * kt
    safe_n = np.where(n > 0.0, n, 1.0)
    g = np.where(n > 0.0, eta * beta_t * (1.0 - beta_t * c) / safe_n, 0.0)
    d_next = r_t[..., None] * d + g[..., None] * a
    return ktil, d_next, c, g


def _defaults(k, beta, r, d0):
    lead = k.shape[:-2]
    Dk = k.shape[-1]
    if r is None:
        r = np.ones(beta.shape, dtype=np.float64)
    if d0 is None:
        d0 = np.ones(lead + (Dk,), dtype=np.float64)
    return r, np.array(d0, dtype=np.float64, copy=True)


def precond_scan_ref(k, beta, r=None, eta=0.1, d0=None):
    """Phase 1 alone: the O(Dk) scan over the key stream.

    [OSDN-it] section 2.2 (two-phase implementation, first phase): produces
    the preconditioned keys {k~_t} and the final preconditioner. Reads only
    k, beta, r, eta and d0.

    Returns (ktilde [B,H,T,Dk], d_T [B,H,Dk], c [B,H,T], g [B,H,T]).
    """
    k, beta, r, d0 = _f64(k), _f64(beta), _f64(r), _f64(d0)
    r, d = _defaults(k, beta, r, d0)
    T = k.shape[-2]
    ktil = np.empty_like(k)
    c_all = np.empty(beta.shape, dtype=np.float64)
    g_all = np.empty(beta.shape, dtype=np.float64)
    for t in range(T):
        kt_, d, c, g = _phase1_step(d, k[..., t, :], beta[..., t], r[..., t], eta)
        ktil[..., t, :] = kt_
        c_all[..., t] = c
        g_all[..., t] = g
    return ktil, d, c_all, g_all


def residual_ratio_ref(k, beta, r=None, eta=0.1, d0=None):
    """Per-token residual contraction ratio and its geometric mean.

    [OSDN-it] section 3 (Theorem 5.2) bounds the product over tokens of the
    ratios f_t(S_t) / f_t(S_{t-1}); for the diagonal update this ratio is
    rho_t = (1 - beta_t <d_t, k_t*k_t>)^2, whatever S_{t-1} and v_t are.
    [OSDN-it] section 4.2 reports the geometric mean of these ratios, q_geo;
    here it is taken per (batch, head) stream over its T tokens,
    q_geo = (prod_t rho_t)^(1/T) = exp(mean_t log rho_t) (1 when T = 0).

    Depends only on the phase-1 inputs. Returns (rho [B,H,T], q_geo [B,H]).
    """
    beta = _f64(beta)
    _, _, c, _ = precond_scan_ref(k, beta, r, eta, d0)
    rho = (1.0 - beta * c) ** 2
    T = rho.shape[-1]
    if T == 0:
        return rho, np.ones(rho.shape[:-1])
    with np.errstate(divide="ignore"):
        q_geo = np.exp(np.mean(np.log(rho), axis=-1))
    return rho, q_geo


# ---------------------------------------------------------------------------
# The full OSDN forward (phase 1 and the memory update, token by token)
# ---------------------------------------------------------------------------

def osdn_ref(q, k, v, beta, r=None, eta=0.1, d0=None, S0=None, scale=1.0,
             return_trace=False, return_states=False):
    """OSDN forward by its token recurrence, fp64.

    Per (batch, head) and token t:
      a = k_t*k_t, n = ||k_t||^2, c = <d_t, a>, k~ = d_t * k_t
      S_t = S_{t-1} + beta_t (v_t - S_{t-1} k_t) k~^T     ([OSDN-it] 2.1)
      o_t = scale * S_t q_t                              (inclusive readout)
      d_{t+1} = r_t d_t + eta beta_t (1 - beta_t c)/n * a ([OSDN-it] 2.2, 2.3)

    Returns (o [B,H,T,Dv], S_T [B,H,Dv,Dk], d_T [B,H,Dk]) and, on request, a
    trace dict with c, g, rho = (1 - beta c)^2 and ktilde, and the list of
    every S_t (S_0 first).
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    r, d = _defaults(k, beta, _f64(r), _f64(d0))
    lead = k.shape[:-2]
    T, Dk = k.shape[-2], k.shape[-1]
    Dv = v.shape[-1]
    if S0 is None:
        S = np.zeros(lead + (Dv, Dk), dtype=np.float64)
    else:
        S = np.array(S0, dtype=np.float64, copy=True)
    o = np.empty(lead + (T, Dv), dtype=np.float64)
    states = [S.copy()] if return_states else None
    if return_trace:
        c_all = np.empty(beta.shape)
        g_all = np.empty(beta.shape)
        ktil_all = np.empty_like(k)
    for t in range(T):
        kt = k[..., t, :]
        bt = beta[..., t]
        ktil, d_next, c, g = _phase1_step(d, kt, bt, r[..., t], eta)
        u = v[..., t, :] - np.einsum("...vk,...k->...v", S, kt)
        S = S + bt[..., None, None] * u[..., :, None] * ktil[..., None, :]
        o[..., t, :] = scale * np.einsum("...vk,...k->...v", S, q[..., t, :])
        if return_trace:
            c_all[..., t] = c
            g_all[..., t] = g
            ktil_all[..., t, :] = ktil
        if return_states:
            states.append(S.copy())
        d = d_next
    out = (o, S, d)
    if return_trace:
        trace = dict(c=c_all, g=g_all, rho=(1.0 - beta * c_all) ** 2,
                     ktilde=ktil_all)
        out = out + (trace,)
    if return_states:
        out = out + (states,)
    return out


def osdn_gated_ref(q, k, v, beta, log_alpha, r=None, eta=0.1, d0=None,
                   S0=None, scale=1.0, return_states=False):
    """OSDN on a gated backbone (per-key-channel decay), token by token, fp64.

    [OSDN-it] section 4 runs OSDN on DeltaNet, Gated DeltaNet and Kimi Delta
    Attention backbones without printing the combined rule. Reading taken:
    the backbone's decay acts on the memory state before the token's delta
    step, and OSDN's step is unchanged, reading with the plain key and
    writing with the preconditioned key; the preconditioner learner (phase 1)
    is untouched:
      S_dec = S_{t-1} Diag(alpha_t)                          (alpha = exp(log_alpha))
      S_t   = S_dec + beta_t (v_t - S_dec k_t) k~_t^T, k~_t = d_t * k_t
      o_t   = scale * S_t q_t
      d_{t+1} as in osdn_ref.
    State [B,H,Dv,Dk] as in osdn_ref (the decay scales the key columns).
    log_alpha: [B,H,T,Dk]; a per-head scalar decay (Gated DeltaNet) is the
    case of equal channels. Returns (o, S_T, d_T) (and every S_t on request).
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    la = _f64(log_alpha)
    r, d = _defaults(k, beta, _f64(r), _f64(d0))
    lead = k.shape[:-2]
    T, Dk = k.shape[-2], k.shape[-1]
    Dv = v.shape[-1]
    S = (np.zeros(lead + (Dv, Dk)) if S0 is None
         else np.array(S0, dtype=np.float64, copy=True))
    o = np.empty(lead + (T, Dv))
    states = [S.copy()] if return_states else None
    for t in range(T):
        kt = k[..., t, :]
        bt = beta[..., t]
        ktil, d_next, _, _ = _phase1_step(d, kt, bt, r[..., t], eta)
        S = S * np.exp(la[..., t, :])[..., None, :]
        u = v[..., t, :] - np.einsum("...vk,...k->...v", S, kt)
        S = S + bt[..., None, None] * u[..., :, None] * ktil[..., None, :]
        o[..., t, :] = scale * np.einsum("...vk,...k->...v", S, q[..., t, :])
        if return_states:
            states.append(S.copy())
        d = d_next
    if return_states:
        return o, S, d, states
    return o, S, d


def deltanet_ref(q, k, v, beta, S0=None, scale=1.0):
    """Plain DeltaNet, S_t = S_{t-1} + beta_t (v_t - S_{t-1} k_t) k_t^T.

    [OSDN-it] section 1: the base recurrence OSDN extends. Readout as in
    osdn_ref. Used by the tests as the d = 1, eta = 0, r = 1 special case.
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    lead = k.shape[:-2]
    T, Dk = k.shape[-2], k.shape[-1]
    Dv = v.shape[-1]
    S = (np.zeros(lead + (Dv, Dk)) if S0 is None
         else np.array(S0, dtype=np.float64, copy=True))
    o = np.empty(lead + (T, Dv))
    for t in range(T):
        kt = k[..., t, :]
        u = v[..., t, :] - np.einsum("...vk,...k->...v", S, kt)
        S = S + beta[..., t, None, None] * u[..., :, None] * kt[..., None, :]
        o[..., t, :] = scale * np.einsum("...vk,...k->...v", S, q[..., t, :])
    return o, S


# ---------------------------------------------------------------------------
# Gated DeltaNet-2
# ---------------------------------------------------------------------------

def gdn2_ref(q, k, v, log_alpha, b, w, S0=None, scale=1.0,
             return_states=False):
    """Gated DeltaNet-2 forward by its token recurrence, fp64.

    [GDN2-it] method, part 1: with erase gate b_t (per key channel), write
    gate w_t (per value channel) and per-channel decay alpha_t,
      S_t = (I - k_t (b_t*k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t*v_t)^T,
    with S of shape [Dk, Dv]. [GDN2-it] method, part 2 (fast-weight view)
    fixes the read orientation: the erase removes the read S^T e_t, e_t =
    b_t*k_t. The output is o_t = scale * S_t^T q_t.

    log_alpha: [B,H,T,Dk] (alpha = exp(log_alpha)); b: [B,H,T,Dk];
    w: [B,H,T,Dv]. Returns (o [B,H,T,Dv], S_T [B,H,Dk,Dv]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    la, b, w = _f64(log_alpha), _f64(b), _f64(w)
    lead = k.shape[:-2]
    T, Dk = k.shape[-2], k.shape[-1]
    Dv = v.shape[-1]
    S = (np.zeros(lead + (Dk, Dv)) if S0 is None
         else np.array(S0, dtype=np.float64, copy=True))
    o = np.empty(lead + (T, Dv))
    states = [S.copy()] if return_states else None
    for t in range(T):
        kt = k[..., t, :]
        S = np.exp(la[..., t, :])[..., :, None] * S
        e = b[..., t, :] * kt
        z = w[..., t, :] * v[..., t, :]
        read = np.einsum("...kv,...k->...v", S, e)
        S = S + kt[..., :, None] * (z - read)[..., None, :]
        o[..., t, :] = scale * np.einsum("...kv,...k->...v", S, q[..., t, :])
        if return_states:
            states.append(S.copy())
    if return_states:
        return o, S, states
    return o, S
