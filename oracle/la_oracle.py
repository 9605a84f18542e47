"""Plain fp64 CPU oracle for the linear-attention baseline the VLA method is measured against.

TEST INFRASTRUCTURE ONLY (same rule as ``vla_oracle.py``): imported by ``tests/``, by
``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py`` only, and it
shares no code with the HIP path.

Source.  The VLA summary (gist.science technical summary of "Variational Linear Attention:
Stable Associative Memory for Long-Context Transformers") describes the method as a
replacement for the unconditional accumulation of standard linear attention (§2.1), with
the output taken, as in standard linear attention, as a ratio of recurrences with the ELU+1
feature map (§2.3, closing paragraph); §1 states that linear attention reaches O(T) through
kernel feature maps and a recurrent state; §2.4 prices the Sherman-Morrison update at about
five times the operations of standard linear attention.  The baseline here is that
standard linear attention with the same feature map and readout, per (batch, head) stream:

  S_0 = 0 (d x d),  n_0 = 0 (d)
  per token t:   S_t = S_{t-1} + v_t phi(k_t)^T
                 n_t = n_{t-1} + phi(k_t)
                 o_t = S_t phi(q_t) / (n_t^T phi(q_t) + eps)
  returns o [.., T, d], S_T [.., d, d], n_T [.., d]

Reading taken: §2.1 prints the accumulation with the raw key; with the ELU+1 feature map
of the readout the accumulated key is phi(k_t), which keeps the ratio's numerator and
denominator consistent (the denominator is the numerator with v replaced by ones).
The loop over t is plain Python over vectorised streams, in float64.
"""

from __future__ import annotations

import numpy as np

from .vla_oracle import phi

__all__ = ["la_forward"]


def la_forward(q, k, v, eps: float = 1e-6, state=None):
    """Linear attention over the second-to-last axis of q, k, v ([..., T, d]).

    ``state`` optionally gives (S_0, n_0) to continue a stream.  Returns (out, S_T, n_T)
    in float64.
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    if not (q.shape == k.shape == v.shape) or q.ndim < 2:
        raise ValueError("q, k, v must share a shape [..., T, d]")
    batch, T, d = q.shape[:-2], q.shape[-2], q.shape[-1]
    if state is None:
        S = np.zeros(batch + (d, d))
        n = np.zeros(batch + (d,))
    else:
        S, n = (np.array(x, dtype=np.float64, copy=True) for x in state)
    out = np.empty(q.shape)
    for t in range(T):
        fk = phi(k[..., t, :])
        fq = phi(q[..., t, :])
        S = S + v[..., t, :, None] * fk[..., None, :]
        n = n + fk
        num = np.matmul(S, fq[..., None])[..., 0]
        out[..., t, :] = num / (np.sum(n * fq, axis=-1) + eps)[..., None]
    return out, S, n
