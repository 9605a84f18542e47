"""Plain fp64 CPU oracle for the Variational Linear Attention (VLA) forward recurrence.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or run this
module: it is used by ``tests/``, by ``__graft_entry__.smoke()`` and by the
``cpu_baseline`` leg of ``bench.py``, and by nothing else.  It shares no code,
constants or helpers with the HIP path.

Source.  "VLA summary" below means the gist.science technical summary of
"Variational Linear Attention: Stable Associative Memory for Long-Context
Transformers" (Pandey & Singh, 2026); the same summary appears on the site's
zh / nl / de / es pages with identical section numbers.

What it computes, for every independent (batch, head) stream (VLA summary §3.2: the
capacity statement is per head, so heads never interact):

  state   A_0 = I / lambda0      (inverse penalty, d x d; M_0 = lambda0 I)
          S_0 = 0                (memory, d_v x d_k, here d x d)
          n_0 = 0                (ELU+1 normaliser, d)
  per token t = 1..T
    khat  = k_t / ||k_t||                                   VLA summary §2.1 / §2.3 (unit keys)
    z     = A_{t-1} u_t                                     §2.3 step 1 (z_t is not defined
    A_t   = A_{t-1} - z z^T / (1 + u_t^T z)                   on the pages; Sherman-Morrison for
                                                            M_t = M_{t-1} + u_t u_t^T, §2.2)
    ahat  = A_t khat / ||A_t khat||                         §2.3 step 2
    S_t   = S_{t-1} + (v_t - S_{t-1} khat) ahat^T           §2.3 step 3
    n_t   = n_{t-1} + phi(k_t)                              §2.3 closing paragraph: output is a
    o_t   = S_t phi(q_t) / (n_t^T phi(q_t) + eps)             ratio of recurrences with the ELU+1
                                                            feature map phi(x) = x+1 (x>0), e^x
  returns o [.., T, d], S_T [.., d, d], A_T [.., d, d]

Readings taken where the pages are silent (each one is also listed in the design notes):
  * u_t is a per-token input used as given (not normalised); z_t = A_{t-1} u_t.
  * A_0 = I/lambda0 with lambda0 > 0 (lambda0 only appears in §3.1, Prop. 2).
  * the readout uses the raw key in phi(k_t), the post-update S_t, and eps outside the dot.
  * zero norms: ||k_t|| = 0 gives khat = 0; ||A_t khat|| = 0 gives ahat = 0 (no S write,
    A still downdates).

Everything is float64; inputs are widened exactly (bf16 / fp32 inputs are representable).
The loop over t is plain Python; streams are vectorised with numpy matmul only.
"""

from __future__ import annotations

import numpy as np

__all__ = ["phi", "init_state", "vla_step", "vla_forward"]


def phi(x: np.ndarray) -> np.ndarray:
    """ELU(x) + 1 with alpha = 1: x + 1 for x > 0, exp(x) otherwise (VLA summary §2.3)."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0.0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def _unit(x: np.ndarray) -> np.ndarray:
    """x / ||x|| along the last axis, with the zero vector mapped to zero."""
    nrm = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    safe = np.where(nrm > 0.0, nrm, 1.0)
    return np.where(nrm > 0.0, x / safe, 0.0)


def init_state(batch_shape, d: int, lambda0: float):
    """(S_0, A_0, n_0) = (0, I/lambda0, 0) for every stream in ``batch_shape``."""
    if not lambda0 > 0.0:
        raise ValueError("lambda0 must be > 0")
    batch_shape = tuple(batch_shape)
    S = np.zeros(batch_shape + (d, d), dtype=np.float64)
    A = np.broadcast_to(np.eye(d) / float(lambda0), batch_shape + (d, d)).copy()
    n = np.zeros(batch_shape + (d,), dtype=np.float64)
    return S, A, n


def vla_step(S, A, n, q_t, k_t, v_t, u_t, eps: float = 1e-6, gain: str = "unit"):
    """One VLA token step for a batch of streams; returns the new state and intermediates.

    S, A: [..., d, d]; n, q_t, k_t, v_t, u_t: [..., d].  ``gain="unit"`` is the method
    (VLA summary §2.3 step 2); ``gain="raw"`` uses A_t khat without the normalisation
    (the ablation discussed with Prop. 2 in §3.1) and is only used to pin the oracle to
    recursive least squares (§5, the RLS connection).
    """
    S = np.asarray(S, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    n = np.asarray(n, dtype=np.float64)
    q_t, k_t, v_t, u_t = (np.asarray(x, dtype=np.float64) for x in (q_t, k_t, v_t, u_t))

    khat = _unit(k_t)
    # §2.3 step 1: Sherman-Morrison downdate of the inverse penalty.
    z = np.matmul(A, u_t[..., None])[..., 0]
    delta = 1.0 + np.sum(u_t * z, axis=-1)
    A_new = A - (z[..., :, None] * z[..., None, :]) / delta[..., None, None]
    # §2.3 step 2: gating vector from the updated A_t.
    y = np.matmul(A_new, khat[..., None])[..., 0]
    if gain == "unit":
        ahat = _unit(y)
    elif gain == "raw":
        ahat = y
    else:
        raise ValueError("gain must be 'unit' or 'raw'")
    # §2.3 step 3: residual update with the pre-update memory S_{t-1}.
    resid = v_t - np.matmul(S, khat[..., None])[..., 0]
    S_new = S + resid[..., :, None] * ahat[..., None, :]
    # §2.3 closing paragraph: ELU+1 ratio readout with the post-update state.
    fq = phi(q_t)
    n_new = n + phi(k_t)
    num = np.matmul(S_new, fq[..., None])[..., 0]
    den = np.sum(n_new * fq, axis=-1) + eps
    o = num / den[..., None]
    return {
        "S": S_new, "A": A_new, "n": n_new, "o": o,
        "khat": khat, "z": z, "delta": delta, "y": y, "ahat": ahat,
        "resid": resid, "den": den,
    }


def vla_forward(q, k, v, u, lambda0: float, eps: float = 1e-6, gain: str = "unit",
                state=None, return_n: bool = False):
    """Run the recurrence over the second-to-last axis of q, k, v, u ([..., T, d]).

    ``state`` optionally gives (S_0, A_0, n_0) to continue a stream (the streaming use of
    VLA summary §5); by default the fixed initial state (0, I/lambda0, 0) is used.
    Returns (out [..., T, d], S_T [..., d, d], A_T [..., d, d]) in float64, plus n_T when
    ``return_n`` is set.
    """
    q, k, v, u = (np.asarray(x, dtype=np.float64) for x in (q, k, v, u))
    if not (q.shape == k.shape == v.shape == u.shape):
        raise ValueError("q, k, v, u must have the same shape [..., T, d]")
    if q.ndim < 2:
        raise ValueError("inputs must be [..., T, d]")
    batch_shape, T, d = q.shape[:-2], q.shape[-2], q.shape[-1]
    if state is None:
        S, A, n = init_state(batch_shape, d, lambda0)
    else:
        S, A, n = (np.array(x, dtype=np.float64, copy=True) for x in state)
    out = np.empty(q.shape, dtype=np.float64)
    for t in range(T):
        r = vla_step(S, A, n, q[..., t, :], k[..., t, :], v[..., t, :], u[..., t, :],
                     eps=eps, gain=gain)
        S, A, n = r["S"], r["A"], r["n"]
        out[..., t, :] = r["o"]
    if return_n:
        return out, S, A, n
    return out, S, A
