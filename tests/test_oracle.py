"""Pins for the fp64 oracle: closed forms, invariants, special cases and brute force.

Each test names the passage of the VLA summary (the gist.science technical summary of
"Variational Linear Attention: Stable Associative Memory for Long-Context Transformers")
that fixes what it checks.  None of them re-types the oracle's own formula: they compare
against a direct inverse, a brute-force minimiser, recursive least squares, the delta
rule, closed forms for d = 1 and T = 1, finite-difference Jacobians and invariances.
"""

import json
import os

import numpy as np
import pytest

from oracle import init_state, phi, vla_forward, vla_step
from oracle.forms import chunked_forward, segment_forward

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(T, d, seed, n=4, scale=1.0):
    rng = np.random.default_rng(seed)
    return [scale * rng.standard_normal((T, d)) for _ in range(n)]


def _trace(q, k, v, u, lam, eps=1e-6, gain="unit"):
    T, d = q.shape
    S, A, n = init_state((), d, lam)
    out = []
    for t in range(T):
        prev = (S, A, n)
        r = vla_step(S, A, n, q[t], k[t], v[t], u[t], eps=eps, gain=gain)
        r["prev"] = prev
        out.append(r)
        S, A, n = r["S"], r["A"], r["n"]
    return out


# --- feature map ----------------------------------------------------------------------

def test_phi_is_elu_plus_one():
    # §2.3: ELU+1 feature map; ELU(x) = x for x > 0, e^x - 1 otherwise (alpha = 1).
    x = np.array([-30.0, -2.0, -1.0, -1e-9, 0.0, 1e-9, 0.5, 3.0])
    expect = np.array([np.exp(-30.0), np.exp(-2.0), np.exp(-1.0), np.exp(-1e-9), 1.0,
                       1.0 + 1e-9, 1.5, 4.0])
    np.testing.assert_allclose(phi(x), expect, rtol=1e-15, atol=0)
    assert np.all(phi(np.linspace(-50, 50, 1001)) > 0)


# --- inverse penalty (§2.2, §2.3 step 1) ----------------------------------------------

@pytest.mark.parametrize("d,lam", [(1, 1.0), (3, 0.5), (8, 2.0)])
def test_A_equals_direct_inverse_of_penalty(d, lam):
    q, k, v, u = _rand(48, d, seed=d)
    M = lam * np.eye(d)
    for t, r in enumerate(_trace(q, k, v, u, lam)):
        M = M + np.outer(u[t], u[t])
        np.testing.assert_allclose(r["A"], np.linalg.inv(M), rtol=1e-9, atol=1e-12)


def test_A_symmetric_positive_definite():
    q, k, v, u = _rand(64, 6, seed=11, scale=3.0)
    for r in _trace(q, k, v, u, 0.5):
        A = r["A"]
        np.testing.assert_allclose(A, A.T, rtol=0, atol=1e-14)
        assert np.linalg.eigvalsh(A).min() > 0
        assert r["delta"] >= 1.0


# --- unit vectors and the residual identity (§2.3) -----------------------------------

def test_unit_key_and_gate():
    q, k, v, u = _rand(40, 5, seed=3)
    for r in _trace(q, k, v, u, 1.0):
        assert abs(np.linalg.norm(r["khat"]) - 1) < 1e-13
        assert abs(np.linalg.norm(r["ahat"]) - 1) < 1e-13
        overlap = r["ahat"] @ r["khat"]
        assert 0 < overlap <= 1 + 1e-14


def test_residual_identity():
    # S_t khat - v = (1 - ahat^T khat)(S_{t-1} khat - v): follows from step 3 and ||khat|| = 1.
    q, k, v, u = _rand(30, 4, seed=5)
    for t, r in enumerate(_trace(q, k, v, u, 0.7)):
        S_prev = r["prev"][0]
        lhs = r["S"] @ r["khat"] - v[t]
        rhs = (1 - r["ahat"] @ r["khat"]) * (S_prev @ r["khat"] - v[t])
        np.testing.assert_allclose(lhs, rhs, rtol=1e-10, atol=1e-12)


# --- brute-force minimiser of the per-step objective (§2.1 "online regularised least
#     squares") ------------------------------------------------------------------------

def _step_objective(S, S_prev, M, beta, khat, v):
    dS = S - S_prev
    r = v - S @ khat
    return beta * (r @ r) + np.trace(dS @ M @ dS.T)


def _quadratic_minimiser(f, d):
    """Minimise a quadratic in vec(S) by probing it: gradient and Hessian from exact
    central differences of f (f is quadratic, so they are exact up to rounding)."""
    n = d * d
    x0 = np.zeros(n)
    h = 1.0
    f0 = f(x0)
    g = np.zeros(n)
    H = np.zeros((n, n))
    E = np.eye(n)
    for i in range(n):
        g[i] = (f(x0 + h * E[i]) - f(x0 - h * E[i])) / (2 * h)
        H[i, i] = (f(x0 + h * E[i]) - 2 * f0 + f(x0 - h * E[i])) / h ** 2
    for i in range(n):
        for j in range(i + 1, n):
            H[i, j] = H[j, i] = (f(x0 + h * E[i] + h * E[j]) - f(x0 + h * E[i] - h * E[j])
                                 - f(x0 - h * E[i] + h * E[j]) + f(x0 - h * E[i] - h * E[j])
                                 ) / (4 * h * h)
    return np.linalg.solve(H, -g)


@pytest.mark.parametrize("T,d,seed", [(8, 4, 0), (6, 3, 1), (8, 2, 2)])
def test_bruteforce_per_step_argmin(T, d, seed):
    """S_t = argmin_S beta_t ||v_t - S khat_t||^2 + tr((S - S_{t-1}) M_t (S - S_{t-1})^T)
    with M_t = lambda0 I + sum u u^T and beta_t = 1 / (||A_t khat|| - khat^T A_t khat):
    the per-step form of the online regularised least squares of §2.1 whose step weight
    gives a unit-norm gain.  M_t, A_t = inv(M_t) and the minimiser are all computed here
    directly (linear solve of the probed quadratic, and separately gradient descent)."""
    lam = 0.8
    q, k, v, u = _rand(T, d, seed=seed)
    M = lam * np.eye(d)
    for t, r in enumerate(_trace(q, k, v, u, lam)):
        M = M + np.outer(u[t], u[t])
        A = np.linalg.inv(M)
        kh = k[t] / np.linalg.norm(k[t])
        Ak = A @ kh
        beta = 1.0 / (np.linalg.norm(Ak) - kh @ Ak)
        S_prev = r["prev"][0]
        f = lambda x: _step_objective(x.reshape(d, d), S_prev, M, beta, kh, v[t])  # noqa: E731
        S_star = _quadratic_minimiser(f, d).reshape(d, d)
        np.testing.assert_allclose(r["S"], S_star, rtol=1e-7, atol=1e-8)
        # plain gradient descent on the same objective, written from its definition
        S = S_prev.copy()
        lip = 2 * (beta + np.linalg.eigvalsh(M).max())
        for _ in range(20000):
            grad = -2 * beta * np.outer(v[t] - S @ kh, kh) + 2 * (S - S_prev) @ M
            S = S - grad / lip
            if np.abs(grad).max() < 1e-13:
                break
        np.testing.assert_allclose(r["S"], S, rtol=1e-7, atol=1e-8)


# --- recursive least squares (§5: the RLS connection) ---------------------------------

def test_rls_special_case_equals_ridge_regression():
    """With u_t = khat_t and the raw gain A_t khat_t the recurrence is textbook RLS, whose
    state is the ridge solution V^T Kh (Kh^T Kh + lambda0 I)^{-1} at every t."""
    T, d, lam = 25, 5, 0.3
    q, k, v, _ = _rand(T, d, seed=9)
    kh = k / np.linalg.norm(k, axis=1, keepdims=True)
    for t, r in enumerate(_trace(q, k, v, kh, lam, gain="raw")):
        K, V = kh[: t + 1], v[: t + 1]
        ridge = V.T @ K @ np.linalg.inv(K.T @ K + lam * np.eye(d))
        np.testing.assert_allclose(r["S"], ridge, rtol=1e-9, atol=1e-11)


# --- special cases --------------------------------------------------------------------

def test_u_zero_is_delta_rule():
    """u = 0 keeps A = I/lambda0, so ahat = khat and the state follows the beta = 1 delta
    rule S_t = S_{t-1}(I - khat khat^T) + v khat^T, which stores v_t exactly (§1, §2.2)."""
    T, d = 20, 6
    q, k, v, _ = _rand(T, d, seed=4)
    u = np.zeros_like(k)
    S = np.zeros((d, d))
    for t, r in enumerate(_trace(q, k, v, u, 2.0)):
        kh = k[t] / np.linalg.norm(k[t])
        S = S @ (np.eye(d) - np.outer(kh, kh)) + np.outer(v[t], kh)
        np.testing.assert_allclose(r["A"], np.eye(d) / 2.0, rtol=0, atol=0)
        np.testing.assert_allclose(r["S"], S, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(r["S"] @ kh, v[t], rtol=1e-12, atol=1e-13)


def test_d1_closed_form():
    """d = 1: khat = ahat = sign(k), so S_t = v_t sign(k_t) and
    o_t = v_t sign(k_t) phi(q_t) / (phi(q_t) sum_{s<=t} phi(k_s) + eps)."""
    T = 50
    rng = np.random.default_rng(7)
    q, k, v, u = (rng.standard_normal((T, 1)) for _ in range(4))
    o, S, A = vla_forward(q, k, v, u, 1.3, eps=1e-6)
    fq = np.where(q > 0, q + 1, np.exp(q))
    fk = np.where(k > 0, k + 1, np.exp(k))
    expect = v * np.sign(k) * fq / (fq * np.cumsum(fk, axis=0) + 1e-6)
    np.testing.assert_allclose(o, expect, rtol=1e-13, atol=0)
    np.testing.assert_allclose(A, [[1.0 / (1.3 + np.sum(u * u))]], rtol=1e-12)


def test_T1_closed_form():
    """T = 1: S_1 = v_1 ahat_1^T, ahat_1 proportional to (lambda0 I + u_1 u_1^T)^{-1} khat_1,
    o_1 = v_1 (ahat_1^T phi(q_1)) / (phi(k_1)^T phi(q_1) + eps)."""
    d, lam = 7, 0.6
    q, k, v, u = _rand(1, d, seed=21)
    o, S, A = vla_forward(q, k, v, u, lam)
    kh = k[0] / np.linalg.norm(k[0])
    g = np.linalg.solve(lam * np.eye(d) + np.outer(u[0], u[0]), kh)
    g = g / np.linalg.norm(g)
    fq = np.where(q[0] > 0, q[0] + 1, np.exp(q[0]))
    fk = np.where(k[0] > 0, k[0] + 1, np.exp(k[0]))
    np.testing.assert_allclose(S, np.outer(v[0], g), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(o[0], v[0] * (g @ fq) / (fk @ fq + 1e-6), rtol=1e-12, atol=1e-14)


def test_hand_worked_example():
    """A one-token example worked by hand in exact arithmetic (tests/golden)."""
    with open(os.path.join(GOLDEN, "hand_t1_d2.json")) as f:
        g = json.load(f)
    arr = lambda key: np.array(g["inputs"][key], dtype=np.float64)[None, :]  # noqa: E731
    o, S, A = vla_forward(arr("q"), arr("k"), arr("v"), arr("u"), g["inputs"]["lambda0"],
                          eps=g["inputs"]["eps"])
    e = g["expected"]
    np.testing.assert_allclose(A, np.array(e["A_num"]) / e["A_den"], rtol=1e-14)
    np.testing.assert_allclose(S, np.array(e["S"]), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(o[0], np.array(e["o_num"]) / e["o_den"], rtol=1e-14)


def test_zero_key_convention():
    """||k_t|| = 0: khat = 0 and ahat = 0, so S is not written; A still downdates; the
    normaliser still gains phi(0) = 1 per component."""
    d = 4
    q, k, v, u = _rand(6, d, seed=8)
    k[3] = 0.0
    tr = _trace(q, k, v, u, 1.0)
    np.testing.assert_array_equal(tr[3]["khat"], 0.0)
    np.testing.assert_array_equal(tr[3]["ahat"], 0.0)
    np.testing.assert_array_equal(tr[3]["S"], tr[2]["S"])
    np.testing.assert_array_equal(tr[3]["n"], tr[2]["n"] + 1.0)
    assert not np.allclose(tr[3]["A"], tr[2]["A"])


# --- invariances, causality, independence ---------------------------------------------

def test_key_scale_invariance():
    q, k, v, u = _rand(30, 5, seed=12)
    o1, S1, A1 = vla_forward(q, k, v, u, 1.0)
    o2, S2, A2 = vla_forward(q, 3.7 * k, v, u, 1.0)
    np.testing.assert_allclose(S2, S1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(A2, A1, rtol=1e-12, atol=1e-15)


def test_penalty_scale_invariance():
    """(lambda0, u) -> (c lambda0, sqrt(c) u) scales M by c: A -> A/c, ahat, S, o unchanged."""
    c = 2.5
    q, k, v, u = _rand(30, 5, seed=13)
    o1, S1, A1 = vla_forward(q, k, v, u, 0.5)
    o2, S2, A2 = vla_forward(q, k, v, np.sqrt(c) * u, 0.5 * c)
    np.testing.assert_allclose(o2, o1, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(S2, S1, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(A2, A1 / c, rtol=1e-11, atol=1e-14)


def test_output_linear_in_values():
    q, k, v, u = _rand(25, 4, seed=14)
    v2 = np.random.default_rng(15).standard_normal(v.shape)
    o1, _, _ = vla_forward(q, k, v, u, 1.0)
    o2, _, _ = vla_forward(q, k, v2, u, 1.0)
    o3, _, _ = vla_forward(q, k, 2.0 * v - 0.5 * v2, u, 1.0)
    np.testing.assert_allclose(o3, 2.0 * o1 - 0.5 * o2, rtol=1e-10, atol=1e-12)


def test_causality():
    q, k, v, u = _rand(20, 4, seed=16)
    o1, _, _ = vla_forward(q, k, v, u, 1.0)
    t0 = 12
    q2, k2, v2, u2 = (x.copy() for x in (q, k, v, u))
    for x in (q2, k2, v2, u2):
        x[t0:] += 1.0
    o2, _, _ = vla_forward(q2, k2, v2, u2, 1.0)
    np.testing.assert_array_equal(o2[:t0], o1[:t0])
    assert not np.allclose(o2[t0:], o1[t0:])


def test_streams_independent_and_batched_equals_single():
    rng = np.random.default_rng(17)
    q, k, v, u = (rng.standard_normal((2, 3, 15, 4)) for _ in range(4))
    o, S, A = vla_forward(q, k, v, u, 0.9)
    perm = [2, 0, 1]
    o_p, S_p, A_p = vla_forward(q[:, perm], k[:, perm], v[:, perm], u[:, perm], 0.9)
    np.testing.assert_array_equal(o_p, o[:, perm])
    for b in range(2):
        for h in range(3):
            o1, S1, A1 = vla_forward(q[b, h], k[b, h], v[b, h], u[b, h], 0.9)
            np.testing.assert_allclose(o[b, h], o1, rtol=1e-14, atol=1e-15)
            np.testing.assert_allclose(S[b, h], S1, rtol=1e-14, atol=1e-15)


# --- Prop. 2 (§3.1), corrected --------------------------------------------------------

def test_jacobian_spectral_radius_is_one():
    """J_t = dS_t / dS_{t-1} by finite differences of the step.  The step is affine in
    S_{t-1}, its transition I - khat ahat^T has eigenvalues 1 (d-1 times) and
    1 - ahat^T khat in [0, 1): spectral radius exactly 1, as Prop. 2 states for the
    normalised case.  The spectral norm is >= 1 and exceeds 1 unless ahat = khat, so the
    radius, not the norm, is what holds exactly."""
    d = 5
    q, k, v, u = _rand(12, d, seed=18)
    for t, r in enumerate(_trace(q, k, v, u, 0.5)):
        S_prev, A_prev, n_prev = r["prev"]
        J = np.zeros((d * d, d * d))
        for i in range(d * d):
            e = np.zeros(d * d)
            e[i] = 1.0
            hi = vla_step(S_prev + e.reshape(d, d), A_prev, n_prev, q[t], k[t], v[t], u[t])
            lo = vla_step(S_prev - e.reshape(d, d), A_prev, n_prev, q[t], k[t], v[t], u[t])
            J[:, i] = ((hi["S"] - lo["S"]) / 2.0).ravel()
        rho = np.abs(np.linalg.eigvals(J)).max()
        assert abs(rho - 1.0) < 1e-9
        assert np.linalg.norm(J, 2) >= 1.0 - 1e-12


# --- Prop. 1 (§3.1): diagnostic only --------------------------------------------------

def test_state_norm_plateaus_diagnostic():
    """||S_t||_F self-limits for bounded inputs while plain linear attention grows (§3.1,
    Prop. 1).  A loose diagnostic, not a parity pin."""
    T, d = 1000, 16
    q, k, v, u = _rand(T, d, seed=19)
    _, S, _ = vla_forward(q, k, v, u, 1.0)
    kh = k / np.linalg.norm(k, axis=1, keepdims=True)
    linear = v.T @ kh
    assert np.linalg.norm(S) < 0.5 * np.linalg.norm(linear)
    assert np.linalg.norm(S) < 4.0 * d


# --- the blocked forms the kernels use ------------------------------------------------

@pytest.mark.parametrize("C", [1, 7, 16, 64])
def test_chunked_form_equals_sequential(C):
    T, d = 200, 16
    q, k, v, u = _rand(T, d, seed=20)
    o, S, A = vla_forward(q, k, v, u, 0.5)
    o2, S2, A2 = chunked_forward(q, k, v, u, 0.5, chunk=C)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-11)
    np.testing.assert_allclose(S2, S, rtol=0, atol=1e-11)
    np.testing.assert_allclose(A2, A, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seg", [1, 50, 64, 77])
def test_segment_form_equals_sequential(seg):
    T, d = 200, 8
    q, k, v, u = _rand(T, d, seed=22)
    o, S, A = vla_forward(q, k, v, u, 0.5)
    o2, S2, A2 = segment_forward(q, k, v, u, 0.5, seg=seg)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-11)
    np.testing.assert_allclose(S2, S, rtol=0, atol=1e-11)
    np.testing.assert_allclose(A2, A, rtol=0, atol=1e-12)


def test_continuation_equals_single_call():
    """Splitting a stream into two calls with the carried (S, A, n) equals one call (the
    streaming use stated in §5)."""
    q, k, v, u = _rand(40, 6, seed=23)
    o, S, A = vla_forward(q, k, v, u, 0.7)
    o1, S1, A1, n1 = vla_forward(q[:17], k[:17], v[:17], u[:17], 0.7, return_n=True)
    o2, S2, A2 = vla_forward(q[17:], k[17:], v[17:], u[17:], 0.7, state=(S1, A1, n1))
    np.testing.assert_allclose(np.concatenate([o1, o2]), o, rtol=0, atol=1e-14)
    np.testing.assert_allclose(S2, S, rtol=0, atol=1e-14)
