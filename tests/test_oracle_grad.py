"""Pins of the gradient oracle (CPU): autograd through the fp64 torch forward against central
finite differences of the numpy oracle, an independent implementation of the forward.

The loss is L = <d_out, out> + <dS_T, S_T> + <dA_T, A_T> + <dn_T, n_T> with random
cotangents.  Every input element of q, k, v, u and lambda0 is perturbed by +-h; the central
difference (L(x + h) - L(x - h)) / 2h has error O(h^2) ~ 1e-10 relative at h = 1e-5.
"""

import numpy as np
import pytest

from oracle import forms, vla_forward, vla_forward_torch, vla_grad


def _loss(q, k, v, u, lam, cot, eps):
    out, S, A, n = vla_forward(q, k, v, u, lam, eps=eps, return_n=True)
    return (np.sum(cot[0] * out) + np.sum(cot[1] * S) + np.sum(cot[2] * A) + np.sum(cot[3] * n))


def _case(N, T, d, seed):
    r = np.random.default_rng(seed)
    x = [r.standard_normal((N, T, d)) for _ in range(4)]
    cot = (r.standard_normal((N, T, d)), r.standard_normal((N, d, d)), r.standard_normal((N, d, d)),
           r.standard_normal((N, d)))
    return x, cot


@pytest.mark.parametrize("N,T,d,lam,seed", [(2, 5, 3, 0.7, 0), (1, 7, 4, 1.5, 1), (1, 3, 2, 0.3, 2)])
def test_gradients_match_finite_differences(N, T, d, lam, seed):
    (q, k, v, u), cot = _case(N, T, d, seed)
    eps = 1e-6
    g = vla_grad(q, k, v, u, lam, cot[0], cot[1], cot[2], cot[3], eps=eps)
    h = 1e-5
    for which in range(4):
        xs = [q, k, v, u]
        fd = np.zeros_like(xs[which])
        for idx in np.ndindex(*xs[which].shape):
            plus = [x.copy() for x in xs]
            minus = [x.copy() for x in xs]
            plus[which][idx] += h
            minus[which][idx] -= h
            fd[idx] = (_loss(*plus, lam, cot, eps) - _loss(*minus, lam, cot, eps)) / (2 * h)
        np.testing.assert_allclose(g[which], fd, rtol=1e-6, atol=1e-7 * np.abs(fd).max())
    # lambda0: one shared value; the oracle returns each stream's share
    fd_lam = (_loss(q, k, v, u, lam + h, cot, eps) - _loss(q, k, v, u, lam - h, cot, eps)) / (2 * h)
    np.testing.assert_allclose(g[4].sum(), fd_lam, rtol=1e-6)


def test_torch_forward_equals_numpy_oracle():
    (q, k, v, u), _ = _case(3, 9, 5, 3)
    import torch
    out, S, A, n = vla_forward_torch(*(torch.tensor(x) for x in (q, k, v, u)),
                                     torch.full((3,), 0.8, dtype=torch.float64))
    ro, rS, rA, rn = vla_forward(q, k, v, u, 0.8, return_n=True)
    for a, b in ((out, ro), (S, rS), (A, rA), (n, rn)):
        np.testing.assert_allclose(a.numpy(), b, rtol=1e-12, atol=1e-14)


def test_planted_mistake_in_the_forward_fails_the_pin():
    """A differentiated forward with one slip (the gate from A_{t-1} instead of A_t) gives
    gradients that disagree with the finite differences of the numpy oracle."""
    import torch
    (q, k, v, u), cot = _case(1, 4, 3, 4)
    tk = torch.tensor(k, requires_grad=True)
    tq, tv, tu = (torch.tensor(x) for x in (q, v, u))
    A = torch.eye(3, dtype=torch.float64)[None] / 0.9
    S = torch.zeros(1, 3, 3, dtype=torch.float64)
    n = torch.zeros(1, 3, dtype=torch.float64)
    loss = 0.0
    for t in range(4):
        kh = tk[:, t] / torch.linalg.norm(tk[:, t], dim=-1, keepdim=True)
        z = torch.einsum("nij,nj->ni", A, tu[:, t])
        A_old = A
        A = A - z[:, :, None] * z[:, None, :] / (1.0 + (tu[:, t] * z).sum(-1))[:, None, None]
        y = torch.einsum("nij,nj->ni", A_old, kh)  # the slip
        ah = y / torch.linalg.norm(y, dim=-1, keepdim=True)
        S = S + (tv[:, t] - torch.einsum("nij,nj->ni", S, kh))[:, :, None] * ah[:, None, :]
        fq = torch.where(tq[:, t] > 0, tq[:, t] + 1.0, torch.exp(torch.clamp(tq[:, t], max=0.0)))
        n = n + torch.where(tk[:, t] > 0, tk[:, t] + 1.0, torch.exp(torch.clamp(tk[:, t], max=0.0)))
        o = torch.einsum("nij,nj->ni", S, fq) / ((n * fq).sum(-1) + 1e-6)[:, None]
        loss = loss + (o * torch.tensor(cot[0][:, t])).sum()
    loss = loss + (S * torch.tensor(cot[1])).sum() + (A * torch.tensor(cot[2])).sum() \
        + (n * torch.tensor(cot[3])).sum()
    loss.backward()
    h = 1e-5
    worst = 0.0
    for idx in np.ndindex(*k.shape):
        plus, minus = k.copy(), k.copy()
        plus[idx] += h
        minus[idx] -= h
        fd = (_loss(q, plus, v, u, 0.9, cot, 1e-6) - _loss(q, minus, v, u, 0.9, cot, 1e-6)) / (2 * h)
        worst = max(worst, abs(tk.grad.numpy()[idx] - fd) / max(1.0, abs(fd)))
    assert worst > 1e-3


@pytest.mark.parametrize("T,seg,d,lam,state", [(23, 8, 4, 0.7, True), (17, 17, 3, 1.3, True),
                                                (25, 6, 5, 0.2, False), (9, 4, 2, 2.0, True)])
def test_segment_backward_form_equals_autograd(T, seg, d, lam, state):
    """The time-segment form of the gradients (the cotangent of A replaced by the suffix sum R,
    the S cotangent through per-segment affine maps, last segments ragged or a single segment)
    equals the autograd oracle, which is itself pinned to finite differences above."""
    r = np.random.default_rng([T, seg, d])
    q, k, v, u, dout = (r.standard_normal((T, d)) for _ in range(5))
    dS = r.standard_normal((d, d)) if state else None
    dA = r.standard_normal((d, d)) if state else None
    dn = r.standard_normal(d) if state else None
    got = forms.segment_backward(q, k, v, u, lam, dout, dS, dA, dn, eps=1e-6, seg=seg)
    ref = vla_grad(q[None], k[None], v[None], u[None], lam, dout[None],
                   None if dS is None else dS[None], None if dA is None else dA[None],
                   None if dn is None else dn[None], eps=1e-6)
    for name, g, rf in zip(("dq", "dk", "dv", "du"), got[:4], ref[:4]):
        assert np.allclose(g, rf[0], rtol=1e-9, atol=1e-9 * np.abs(rf[0]).max()), name
    assert abs(got[4] - ref[4][0]) <= 1e-9 * max(1.0, abs(ref[4][0]))
