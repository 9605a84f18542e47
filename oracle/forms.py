"""Second formulations of the VLA recurrence, in fp64, for pinning the algebra the GPU uses.

TEST INFRASTRUCTURE ONLY (same rule as ``oracle/vla_oracle.py``): imported by ``tests/``
only.  The recurrence itself is in ``vla_oracle.py``; the functions here re-derive the same
results in the blocked forms the kernels are built on (the forward in chunks and in time
segments, and the gradients in time segments), and the tests check them against the
sequential oracle and the autograd oracle before any kernel is trusted.  The pages name a parallel
scan formulation but give no detail (VLA summary §2.4); the blocked forms below are
derived from the recurrence of §2.3 with the Woodbury identity and the UT/WY transform.

Notation for one chunk of m tokens starting from (A0, S0, n0); rows of U, Kh, V, Fq, Fk
are u_j, khat_j, v_j, phi(q_j), phi(k_j):

  Z0 = U A0                      G = I + Z0 U^T = L D L^T   (L unit lower, D = diag(delta))
  Z  = L^{-1} Z0                 row j is the sequential z_j = A_{j-1} u_j, D_jj = delta_j
  Y  = Kh A0 - tril0(Kh Z^T) D^{-1} Z      row j is A_j khat_j
  ahat_j = Y_j / ||Y_j||         A_end = A0 - Z^T D^{-1} Z
  Tm = (I + tril-1(Kh ahat^T))^{-1}
  E  = Tm (V - Kh S0^T)          row j is e_j = v_j - S_{j-1} khat_j
  S_end = S0 + E^T ahat          Num = Fq S0^T + tril0(Fq ahat^T) E
  den_j = phi(q_j)^T (n0 + sum_{i<=j} phi(k_i)) + eps

tril0 keeps the diagonal, tril-1 is strictly lower.  The segment form uses the two facts
that A_t = (lambda0 I + sum_{s<=t} u_s u_s^T)^{-1} is a function of a prefix sum, and that
the S recurrence is affine: S_b = S_a Pi + B with Pi = prod (I - khat ahat^T).
"""

from __future__ import annotations

import numpy as np

from .vla_oracle import phi

__all__ = ["ldl_unit_lower", "chunk_step", "chunked_forward", "segment_forward", "segment_backward"]


def _unit_rows(x):
    nrm = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return np.where(nrm > 0.0, x / np.where(nrm > 0.0, nrm, 1.0), 0.0)


def ldl_unit_lower(G):
    """G = L diag(D) L^T for a symmetric positive definite G (plain column algorithm)."""
    m = G.shape[0]
    L = np.eye(m)
    D = np.zeros(m)
    for j in range(m):
        D[j] = G[j, j] - np.sum(L[j, :j] ** 2 * D[:j])
        for i in range(j + 1, m):
            L[i, j] = (G[i, j] - np.sum(L[i, :j] * L[j, :j] * D[:j])) / D[j]
    return L, D


def chunk_step(A0, S0, n0, q, k, v, u, eps=1e-6):
    """Advance one stream over one chunk (rows of q, k, v, u) in the blocked form."""
    m = q.shape[0]
    Kh = _unit_rows(k)
    Fq, Fk = phi(q), phi(k)
    Z0 = u @ A0
    G = np.eye(m) + Z0 @ u.T
    L, D = ldl_unit_lower(G)
    Z = np.linalg.solve(L, Z0)
    Y = Kh @ A0 - (np.tril(Kh @ Z.T) / D[None, :]) @ Z
    ahat = _unit_rows(Y)
    A_end = A0 - Z.T @ (Z / D[:, None])
    Tm = np.linalg.inv(np.eye(m) + np.tril(Kh @ ahat.T, -1))
    E = Tm @ (v - Kh @ S0.T)
    S_end = S0 + E.T @ ahat
    num = Fq @ S0.T + np.tril(Fq @ ahat.T) @ E
    ncum = n0[None, :] + np.cumsum(Fk, axis=0)
    den = np.sum(Fq * ncum, axis=1) + eps
    return num / den[:, None], S_end, A_end, ncum[-1]


def chunked_forward(q, k, v, u, lambda0, eps=1e-6, chunk=64):
    """Single stream [T, d]; returns (out, S_T, A_T) computed chunk by chunk."""
    q, k, v, u = (np.asarray(x, dtype=np.float64) for x in (q, k, v, u))
    T, d = q.shape
    A, S, n = np.eye(d) / lambda0, np.zeros((d, d)), np.zeros(d)
    out = np.empty((T, d))
    for a in range(0, T, chunk):
        b = min(T, a + chunk)
        o, S, A, n = chunk_step(A, S, n, q[a:b], k[a:b], v[a:b], u[a:b], eps)
        out[a:b] = o
    return out, S, A


def segment_forward(q, k, v, u, lambda0, eps=1e-6, seg=64):
    """Single stream [T, d], segments of ``seg`` tokens processed independently.

    A at each segment start is the direct inverse of lambda0 I + (Gram of all earlier
    u); each segment then yields its affine map S_end = S_start Pi + B (from S_start = I
    and S_start = 0 with v), the maps are composed in order, and the outputs are
    recomputed from the true segment start.
    """
    q, k, v, u = (np.asarray(x, dtype=np.float64) for x in (q, k, v, u))
    T, d = q.shape
    starts = list(range(0, T, seg))
    gram_prefix = np.zeros((d, d))
    nk_prefix = np.zeros(d)
    seg_in = []
    for a in starts:
        b = min(T, a + seg)
        A_start = np.linalg.inv(lambda0 * np.eye(d) + gram_prefix)
        seg_in.append((a, b, A_start, nk_prefix.copy()))
        gram_prefix = gram_prefix + u[a:b].T @ u[a:b]
        nk_prefix = nk_prefix + phi(k[a:b]).sum(axis=0)
    # per segment: gating vectors from A_start, then the affine map of S.
    maps = []
    for a, b, A_start, _ in seg_in:
        A = A_start.copy()
        Kh = _unit_rows(k[a:b])
        ahat = np.empty((b - a, d))
        for j in range(b - a):
            z = A @ u[a + j]
            A = A - np.outer(z, z) / (1.0 + u[a + j] @ z)
            ahat[j] = _unit_rows((A @ Kh[j])[None, :])[0]
        Pi, B = np.eye(d), np.zeros((d, d))
        for j in range(b - a):
            Pi = Pi - np.outer(Pi @ Kh[j], ahat[j])
            B = B + np.outer(v[a + j] - B @ Kh[j], ahat[j])
        maps.append((Pi, B, ahat, A))
    out = np.empty((T, d))
    S = np.zeros((d, d))
    for (a, b, _, n0), (Pi, B, ahat, A_end) in zip(seg_in, maps):
        Kh = _unit_rows(k[a:b])
        Fq, Fk = phi(q[a:b]), phi(k[a:b])
        Sx = S.copy()
        n = n0.copy()
        for j in range(b - a):
            Sx = Sx + np.outer(v[a + j] - Sx @ Kh[j], ahat[j])
            n = n + Fk[j]
            out[a + j] = Sx @ Fq[j] / (n @ Fq[j] + eps)
        S = S @ Pi + B
    return out, S, maps[-1][3]


def segment_backward(q, k, v, u, lambda0, d_out, dS_T=None, dA_T=None, dn_T=None, eps=1e-6, seg=64):
    """Gradients (dq, dk, dv, du [T, d], dlambda0) of
    L = <d_out, out> + <dS_T, S_T> + <dA_T, A_T> + <dn_T, n_T>  for one stream [T, d], in
    time segments of ``seg`` tokens: the form the segment-parallel backward kernels follow.

    * The cotangent of A_t is never formed.  A_t = (lambda0 I + sum_{s<=t} u_s u_s^T)^{-1}
      (Sherman-Morrison keeps it exactly, VLA summary §2.2) reaches the loss only through
      y_t = A_t khat_t and through A_T, and d(X^{-1}) = -X^{-1} dX X^{-1}; so with
      w_t = A_t dy_t and R_s = sum_{t>=s} (w_t y_t^T + y_t w_t^T) / 2 + A_T sym(dA_T) A_T,
          du_s = -2 R_s u_s,      dlambda0 = -tr R_0.
    * The cotangent of S obeys dS_{t-1} = (dS_t + dnum_t phi(q_t)^T)(I - ahat_t khat_t^T):
      affine in dS_t with coefficients fixed by the forward, so each segment maps the
      cotangent E at its end to  E Lm + Bm  at its start; the maps compose from the last
      segment back.  dn is a suffix sum of dden_t phi(q_t); R a suffix sum over segments.
    * Each segment is then swept from its end with the true dS and dn, R local to the
      segment, and du is completed with -2 R_end u over the segment's tokens.
    """
    q, k, v, u, d_out = (np.asarray(x, dtype=np.float64) for x in (q, k, v, u, d_out))
    T, d = q.shape
    dS_T = np.zeros((d, d)) if dS_T is None else np.asarray(dS_T, dtype=np.float64)
    dA_T = np.zeros((d, d)) if dA_T is None else np.asarray(dA_T, dtype=np.float64)
    dn_T = np.zeros(d) if dn_T is None else np.asarray(dn_T, dtype=np.float64)
    dphi = lambda x: np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0)))
    bounds = [(a, min(T, a + seg)) for a in range(0, T, seg)]
    P = len(bounds)
    # forward per segment from its start state (the start states by a plain forward), keeping
    # each token's quantities and the state after it
    S, A, n = np.zeros((d, d)), np.eye(d) / lambda0, np.zeros(d)
    recs = []
    for a, b in bounds:
        rs = []
        for t in range(a, b):
            rk = 1.0 / np.linalg.norm(k[t])
            kh = k[t] * rk
            z = A @ u[t]
            A = A - np.outer(z, z) / (1.0 + u[t] @ z)
            y = A @ kh
            yn = np.linalg.norm(y)
            ah = y / yn
            r = v[t] - S @ kh
            S_prev = S
            S = S + np.outer(r, ah)
            n = n + phi(k[t])
            fq = phi(q[t])
            den = n @ fq + eps
            rs.append(dict(kh=kh, ah=ah, y=y, yn=yn, rk=rk, r=r, fq=fq, den=den, o=S @ fq / den,
                           S=S, S_prev=S_prev, A=A, n=n))
        recs.append(rs)
    A_T = A
    # segment maps of the S cotangent and segment sums of dden phi(q) (not needed for the
    # first segment)
    Lm, Bm, nd = [None] * P, [None] * P, [None] * P
    for p in range(1, P):
        a, _ = bounds[p]
        L, B, ndp = np.eye(d), np.zeros((d, d)), np.zeros(d)
        for j in reversed(range(len(recs[p]))):
            rc, t = recs[p][j], a + j
            ndp = ndp - (d_out[t] @ rc["o"]) / rc["den"] * rc["fq"]
            B = B + np.outer(d_out[t] / rc["den"], rc["fq"])
            B = B - np.outer(B @ rc["ah"], rc["kh"])
            L = L - np.outer(L @ rc["ah"], rc["kh"])
        Lm[p], Bm[p], nd[p] = L, B, ndp
    # the cotangents at every segment end, from the last segment back
    E, dn_end = [None] * P, [None] * P
    E[P - 1], dn_end[P - 1] = dS_T, dn_T
    for p in range(P - 1, 0, -1):
        E[p - 1] = E[p] @ Lm[p] + Bm[p]
        dn_end[p - 1] = dn_end[p] + nd[p]
    # per segment, from its end: gradients with R local to the segment
    dq, dk, dv, du = (np.zeros((T, d)) for _ in range(4))
    W, trace = [None] * P, 0.0
    for p in range(P):
        a, _ = bounds[p]
        dS, dn, R = E[p].copy(), dn_end[p].copy(), np.zeros((d, d))
        for j in reversed(range(len(recs[p]))):
            rc, t = recs[p][j], a + j
            dden = -(d_out[t] @ rc["o"]) / rc["den"]
            dnum = d_out[t] / rc["den"]
            dS = dS + np.outer(dnum, rc["fq"])
            dq[t] = (rc["S"].T @ dnum + dden * rc["n"]) * dphi(q[t])
            dn = dn + dden * rc["fq"]
            dr = dS @ rc["ah"]
            dah = dS.T @ rc["r"]
            dv[t] = dr
            dy = (dah - rc["ah"] * (rc["ah"] @ dah)) / rc["yn"]
            dS = dS - np.outer(dr, rc["kh"])
            w = rc["A"] @ dy
            dkh = w - rc["S_prev"].T @ dr
            R = R + 0.5 * (np.outer(w, rc["y"]) + np.outer(rc["y"], w))
            trace += w @ rc["y"]
            du[t] = -2.0 * R @ u[t]
            dk[t] = (dkh - rc["kh"] * (rc["kh"] @ dkh)) * rc["rk"] + dn * dphi(k[t])
        W[p] = R
    # R at every segment end (suffix sums after the final-state term) completes du
    X = A_T @ (0.5 * (dA_T + dA_T.T)) @ A_T
    R_end = X.copy()
    for p in range(P - 1, -1, -1):
        a, b = bounds[p]
        du[a:b] -= 2.0 * u[a:b] @ R_end
        R_end = R_end + W[p]
    dlambda0 = -(trace + np.trace(X))
    return dq, dk, dv, du, dlambda0
