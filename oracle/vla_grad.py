"""fp64 CPU oracle for the gradients of the VLA forward recurrence (test infrastructure only).

TEST INFRASTRUCTURE ONLY (same rule as ``vla_oracle.py``): imported by ``tests/`` only; it
shares no code with the HIP path.

The forward below is the recurrence of VLA summary §2.3 (same steps and order as
``vla_oracle.vla_step``: unit key, Sherman-Morrison downdate with z = A_{t-1} u_t, unit gate
from A_t, residual update with S_{t-1}, ELU+1 ratio readout with the post-update state),
written with torch float64 CPU tensors so that autograd, a library primitive, differentiates
it.  The gradient of a scalar loss

    L = sum(d_out * out) + sum(dS_T * S_T) + sum(dA_T * A_T) + sum(dn_T * n_T)

is returned for q, k, v, u and for lambda0 (per stream: each stream's own A_0 = I / lambda0,
so the total derivative is the sum over streams).  The tests pin it to central finite
differences of the numpy oracle, an independent implementation of the forward.
Zero norms (||k|| = 0 or ||A_t khat|| = 0) have no derivative; they are not used here.

``dtype`` is float64 for the oracle.  The same steps evaluated in float32 (``dtype=
torch.float32``) are not a reference: they measure how far plain fp32 arithmetic of this
recurrence strays from the fp64 gradients on a given input (some gradients, e.g. du where
u_t = k_t, are ill-conditioned), which sets the tolerance the fp32 kernels are held to.
"""

from __future__ import annotations

import numpy as np
import torch

__all__ = ["vla_forward_torch", "vla_grad"]


def _phi(x):
    return torch.where(x > 0, x + 1.0, torch.exp(torch.clamp(x, max=0.0)))


def vla_forward_torch(q, k, v, u, lam, eps: float = 1e-6):
    """q, k, v, u: [N, T, d] float64 tensors; lam: [N] float64.  Returns out, S_T, A_T, n_T."""
    N, T, d = q.shape
    eye = torch.eye(d, dtype=q.dtype)
    A = eye.expand(N, d, d) / lam[:, None, None]
    S = torch.zeros(N, d, d, dtype=q.dtype)
    n = torch.zeros(N, d, dtype=q.dtype)
    outs = []
    for t in range(T):
        kt, ut, vt, qt = k[:, t], u[:, t], v[:, t], q[:, t]
        kh = kt / torch.linalg.norm(kt, dim=-1, keepdim=True)
        z = torch.einsum("nij,nj->ni", A, ut)
        delta = 1.0 + (ut * z).sum(-1)
        A = A - z[:, :, None] * z[:, None, :] / delta[:, None, None]
        y = torch.einsum("nij,nj->ni", A, kh)
        ah = y / torch.linalg.norm(y, dim=-1, keepdim=True)
        r = vt - torch.einsum("nij,nj->ni", S, kh)
        S = S + r[:, :, None] * ah[:, None, :]
        fq = _phi(qt)
        n = n + _phi(kt)
        num = torch.einsum("nij,nj->ni", S, fq)
        outs.append(num / ((n * fq).sum(-1) + eps)[:, None])
    return torch.stack(outs, dim=1), S, A, n


def vla_grad(q, k, v, u, lambda0, d_out, dS_T=None, dA_T=None, dn_T=None, eps: float = 1e-6,
             dtype=torch.float64):
    """Gradients (dq, dk, dv, du [N, T, d], dlambda0 [N]) of the loss above, as float64 numpy
    arrays; inputs are [N, T, d] arrays (N independent streams)."""
    tq, tk, tv, tu = (torch.tensor(np.asarray(x, dtype=np.float64), dtype=dtype, requires_grad=True)
                      for x in (q, k, v, u))
    N = tq.shape[0]
    lam = torch.full((N,), float(lambda0), dtype=dtype, requires_grad=True)
    out, S, A, n = vla_forward_torch(tq, tk, tv, tu, lam, eps=eps)
    loss = (out * torch.tensor(np.asarray(d_out, dtype=np.float64), dtype=dtype)).sum()
    for state, cot in ((S, dS_T), (A, dA_T), (n, dn_T)):
        if cot is not None:
            loss = loss + (state * torch.tensor(np.asarray(cot, dtype=np.float64), dtype=dtype)).sum()
    loss.backward()
    return tuple(x.grad.double().numpy() for x in (tq, tk, tv, tu, lam))
