"""Exact rational versions of the recurrences, for tiny inputs.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Inputs are nested lists (or arrays) of ``fractions.Fraction``/ints. Keys are
not normalised, so no square root is needed and every quantity stays rational.
Two independent computations are offered for each method:

* the token recurrence itself, exactly ("step" functions), and
* the closed-form unrolling of the linear state recurrence as products of
  transition matrices ("unrolled" functions).

They are written separately (matrix products versus rank-one updates) so that
an index or order mistake in one does not reproduce in the other.
"""

from fractions import Fraction


def _F(x):
    return x if isinstance(x, Fraction) else Fraction(x)


def _vec(x):
    return [_F(e) for e in x]


def _mat(x):
    return [[_F(e) for e in row] for row in x]


def _zeros(m, n):
    return [[Fraction(0)] * n for _ in range(m)]


def _eye(n):
    return [[Fraction(int(i == j)) for j in range(n)] for i in range(n)]


def _matmul(A, B):
    n, m, p = len(A), len(B), len(B[0])
    return [[sum((A[i][l] * B[l][j] for l in range(m)), Fraction(0))
             for j in range(p)] for i in range(n)]


def _matvec(A, x):
    return [sum((A[i][j] * x[j] for j in range(len(x))), Fraction(0))
            for i in range(len(A))]


def _dot(x, y):
    return sum((a * b for a, b in zip(x, y)), Fraction(0))


def _outer(x, y):
    return [[a * b for b in y] for a in x]


def _add(A, B):
    return [[a + b for a, b in zip(ra, rb)] for ra, rb in zip(A, B)]


# ---------------------------------------------------------------------------
# OSDN
# ---------------------------------------------------------------------------

def osdn_exact(q, k, v, beta, r, eta, d0, S0):
    """Exact OSDN token recurrence for one (batch, head).

    q, k: T x Dk; v: T x Dv; beta, r: length T; d0: Dk; S0: Dv x Dk.
    Same equations as ``recurrence.osdn_ref`` ([OSDN-it] sections 2.1-2.3,
    descent sign), in rationals. Returns (o, S_T, d_T, ktilde, states) with
    states = [S_0, S_1, ..., S_T].
    """
    eta = _F(eta)
    d = _vec(d0)
    S = _mat(S0)
    o, ktil, states = [], [], [S]
    for t in range(len(k)):
        kt, vt, qt = _vec(k[t]), _vec(v[t]), _vec(q[t])
        bt, rt = _F(beta[t]), _F(r[t])
        a = [x * x for x in kt]
        n = sum(a, Fraction(0))
        c = _dot(d, a)
        kti = [di * ki for di, ki in zip(d, kt)]
        ktil.append(kti)
        u = [vi - si for vi, si in zip(vt, _matvec(S, kt))]
        S = _add(S, _outer([bt * ui for ui in u], kti))
        states.append(S)
        o.append(_matvec(S, qt))
        g = eta * bt * (1 - bt * c) / n if n != 0 else Fraction(0)
        d = [rt * di + g * ai for di, ai in zip(d, a)]
    return o, S, d, ktil, states


def osdn_unrolled_state(k, v, beta, ktil, S0):
    """S_T from the explicit product form of the linear state recurrence.

    Rewriting the [OSDN-it] section 2.1 update as
    S_t = S_{t-1} (I - beta_t k_t k~_t^T) + beta_t v_t k~_t^T gives
    S_T = S_0 M_1 ... M_T + sum_t beta_t v_t k~_t^T M_{t+1} ... M_T,
    with M_t = I - beta_t k_t k~_t^T. Computed by matrix products, right to
    left, independently of ``osdn_exact``.
    """
    T = len(k)
    Dk = len(k[0])
    Ms = []
    for t in range(T):
        bt = _F(beta[t])
        kk = _outer(_vec(k[t]), _vec(ktil[t]))
        Ms.append([[Fraction(int(i == j)) - bt * kk[i][j] for j in range(Dk)]
                   for i in range(Dk)])
    # suffix products P_t = M_{t+1} ... M_T (P_T = I)
    suffix = [None] * (T + 1)
    suffix[T] = _eye(Dk)
    for t in range(T - 1, -1, -1):
        suffix[t] = _matmul(Ms[t], suffix[t + 1])
    S = _matmul(_mat(S0), suffix[0])
    for t in range(T):
        bt = _F(beta[t])
        w = _outer([bt * x for x in _vec(v[t])], _vec(ktil[t]))
        S = _add(S, _matmul(w, suffix[t + 1]))
    return S


def precond_unrolled(k, beta, r, eta, d0):
    """Phase-1 preconditioner after T tokens, as an affine-map product.

    Substituting g_t into the [OSDN-it] section 2.3 update (descent sign)
    gives the affine map d_{t+1} = (r_t I - rho_t a_t a_t^T) d_t + e_t a_t with
    a_t = k_t*k_t, rho_t = eta beta_t^2/||k_t||^2, e_t = eta beta_t/||k_t||^2.
    Composes the T maps as matrices (independently of ``osdn_exact``) and
    returns (d_{T+1}, [d_1, ..., d_{T+1}]).
    """
    eta = _F(eta)
    Dk = len(d0)
    d = _vec(d0)
    ds = [d]
    for t in range(len(k)):
        kt = _vec(k[t])
        a = [x * x for x in kt]
        n = sum(a, Fraction(0))
        bt, rt = _F(beta[t]), _F(r[t])
        if n == 0:
            F = [[rt * int(i == j) for j in range(Dk)] for i in range(Dk)]
            e = [Fraction(0)] * Dk
        else:
            rho = eta * bt * bt / n
            F = [[rt * int(i == j) - rho * a[i] * a[j] for j in range(Dk)]
                 for i in range(Dk)]
            e = [eta * bt / n * ai for ai in a]
        d = [x + y for x, y in zip(_matvec(F, d), e)]
        ds.append(d)
    return d, ds


# ---------------------------------------------------------------------------
# GDN-2
# ---------------------------------------------------------------------------

def gdn2_exact(q, k, v, alpha, b, w, S0):
    """Exact GDN-2 token recurrence for one (batch, head).

    [GDN2-it] method part 1, S of shape Dk x Dv; alpha is given directly
    (rational) instead of its logarithm. Returns (o, S_T, states).
    """
    S = _mat(S0)
    states = [S]
    o = []
    for t in range(len(k)):
        kt, vt, qt = _vec(k[t]), _vec(v[t]), _vec(q[t])
        al, bt, wt = _vec(alpha[t]), _vec(b[t]), _vec(w[t])
        Sd = [[al[i] * S[i][j] for j in range(len(S[0]))] for i in range(len(S))]
        e = [x * y for x, y in zip(bt, kt)]
        z = [x * y for x, y in zip(wt, vt)]
        read = [sum((Sd[i][j] * e[i] for i in range(len(e))), Fraction(0))
                for j in range(len(S[0]))]
        S = _add(Sd, _outer(kt, [zi - ri for zi, ri in zip(z, read)]))
        states.append(S)
        o.append([sum((S[i][j] * qt[i] for i in range(len(qt))), Fraction(0))
                  for j in range(len(S[0]))])
    return o, S, states


def gdn2_unrolled_state(k, v, alpha, b, w, S0):
    """GDN-2 S_T as N_T ... N_1 S_0 + sum_t N_T ... N_{t+1} k_t z_t^T.

    N_t = (I - k_t e_t^T) Diag(alpha_t), e_t = b_t*k_t, z_t = w_t*v_t
    ([GDN2-it] method part 1), composed by matrix products.
    """
    T = len(k)
    Dk = len(k[0])
    Ns = []
    for t in range(T):
        kt = _vec(k[t])
        e = [x * y for x, y in zip(_vec(b[t]), kt)]
        al = _vec(alpha[t])
        Ns.append([[(int(i == j) - kt[i] * e[j]) * al[j] for j in range(Dk)]
                   for i in range(Dk)])
    # prefix-from-the-left products L_t = N_T ... N_{t+1}
    left = [None] * (T + 1)
    left[T] = _eye(Dk)
    for t in range(T - 1, -1, -1):
        left[t] = _matmul(left[t + 1], Ns[t])
    S = _matmul(left[0], _mat(S0))
    for t in range(T):
        z = [x * y for x, y in zip(_vec(w[t]), _vec(v[t]))]
        S = _add(S, _matmul(left[t + 1], _outer(_vec(k[t]), z)))
    return S
