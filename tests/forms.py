"""Independent fp64 formulations of the gated delta rule, used to pin the oracle.

Neither of these is the oracle: each reaches the same result by a different
route, so a dropped term, a wrong sign, a transposed state or a wrong index in
the oracle shows up as a disagreement.

* ``unrolled``: the closed unrolled form of the recurrence.  With transition
  A_m = a_m (I - b_m k_m k_m^T), the state after t tokens is
      S_t = S_0 A_1 ... A_t + sum_j b_j v_j k_j^T A_{j+1} ... A_t,
  so o_t = scale * S_t q_t is evaluated right to left on vectors, O(T^2 d).
* ``chunked``: the chunk (WY / UT transform) form.  Inside a chunk with
  G = inclusive cumsum of g, gamma = exp(G), E_ij = exp(G_i - G_j):
      A = strict_lower(diag(b) E * K K^T),  (I + A) U = diag(b) V - diag(b gamma) K S0^T,
      O = scale (diag(gamma) Q S0^T + lower(E * Q K^T) U),
      S_L = gamma_L S0 + U^T diag(exp(G_L - G)) K.
  The triangular solve is scipy's.
Both take one value head: q, k [T, dk]; v [T, dv]; g, b [T]; S0 [dv, dk].
"""
import numpy as np
from scipy.linalg import solve_triangular


def unrolled(q, k, v, g, b, S0, scale=1.0):
    T, dk = q.shape
    dv = v.shape[1]
    a = np.exp(g)
    o = np.zeros((T, dv))
    for t in range(T):
        w = q[t].copy()              # w = A_{j+1} ... A_t q_t, built from j = t downwards
        acc = np.zeros(dv)
        for j in range(t, -1, -1):
            acc += b[j] * v[j] * (k[j] @ w)
            w = a[j] * (w - b[j] * k[j] * (k[j] @ w))   # w <- A_j w
        acc += S0 @ w
        o[t] = scale * acc
    # final state: S_T = S0 P + sum_j b_j v_j (k_j^T A_{j+1..T}), rows of P via transposes
    M = np.eye(dk)
    ST = np.zeros((dv, dk))
    for j in range(T - 1, -1, -1):
        ST += b[j] * np.outer(v[j], k[j] @ M)
        M = a[j] * (M - b[j] * np.outer(k[j], k[j] @ M))   # M <- A_j M
    ST += S0 @ M
    return o, ST


def chunked(q, k, v, g, b, S0, chunk=64, scale=1.0):
    T, dk = q.shape
    dv = v.shape[1]
    S = S0.astype(np.float64).copy()
    o = np.zeros((T, dv))
    for c0 in range(0, T, chunk):
        sl = slice(c0, min(c0 + chunk, T))
        K, Q, V, gc, bc = k[sl], q[sl], v[sl], g[sl], b[sl]
        L = K.shape[0]
        G = np.cumsum(gc)
        gam = np.exp(G)
        E = np.exp(G[:, None] - G[None, :])
        A = np.tril(bc[:, None] * E * (K @ K.T), -1)
        rhs = bc[:, None] * V - (bc * gam)[:, None] * (K @ S.T)
        U = solve_triangular(np.eye(L) + A, rhs, lower=True, unit_diagonal=True)
        P = np.tril(E * (Q @ K.T))
        o[sl] = scale * (gam[:, None] * (Q @ S.T) + P @ U)
        S = gam[-1] * S + (np.exp(G[-1] - G)[:, None] * U).T @ K
    return o, S


def heads(q, k, v, g, b, h0, n, h, group):
    """Slice one (sequence-less) value head h out of [T, H, d] tensors as fp64."""
    kh = h // group
    S0 = np.zeros((v.shape[2], q.shape[2])) if h0 is None else h0[n, h]
    return q[:, kh], k[:, kh], v[:, h], g[:, h], b[:, h], S0
