"""The un-normalised-gain ablation (gain A_t khat instead of ahat) against the fp64 oracle,
and the state-transition product it is measured with (GPU only).

The oracle's raw gain is pinned on the CPU by the recursive-least-squares special case.
With v = 0 and S_0 = I the recurrence leaves S_T = J_1 J_2 ... J_T, J_t = I - khat_t g_t^T,
so the same calls measure the product whose norm the ablation reports.
Bars as for the method: relative L2 < 1e-4 (fp32 inputs), < 1e-2 (bf16 inputs).
"""

import sys

import numpy as np
import pytest
import torch

from rls_associative_memory_amd import vla
from rls_associative_memory_amd.inputs import get_workload, make_inputs, torch_dtype

from .parity import TOL, rel_l2
from oracle import vla_forward as oracle_forward

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _dev(x, w, shape):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).view(shape).to(
        torch_dtype(w)).cuda()


def _rounded(w, arrays):
    if w.dtype == "bf16":
        return [torch.from_numpy(x).to(torch.bfloat16).float().numpy() for x in arrays]
    return list(arrays)


def _compare(label, tol, got, ref):
    names = ("out", "S", "A", "n")
    errs = {n: rel_l2(g, r) for n, g, r in zip(names, got, ref)}
    _say(f"[parity] {label}: " + " ".join(f"{n}={e:.3e}" for n, e in errs.items()) + f" (tol {tol:g})")
    for n, e in errs.items():
        assert e < tol, f"{label}: {n} rel L2 {e:.3e} >= {tol:g}"


@pytest.mark.parametrize("d", [32, 64, 96, 128])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_raw_gain_matches_oracle(d, dt):
    T, H = 200, 3
    w = get_workload("tiny_t256_d32").resized(name=f"raw_{d}_{dt}", B=1, H=H, T=T, d=d, dtype=dt,
                                              lambda0=2.0)
    q, k, v, u = _rounded(w, make_inputs(w))
    ref = oracle_forward(q, k, v, u, w.lambda0, eps=w.eps, gain="raw", return_n=True)
    dev = [_dev(x, w, (1, H, T, d)) for x in (q, k, v, u)]
    _say(f"[case] raw gain d={d} {dt} T={T}")
    out, S, A, n = vla.forward_state(*dev, w.lambda0, eps=w.eps, gain="raw")  # auto: sequential
    torch.cuda.synchronize()
    got = (_np(out).reshape(H, T, d), _np(S).reshape(H, d, d), _np(A).reshape(H, d, d),
           _np(n).reshape(H, d))
    _compare(f"raw gain d={d} {dt}", TOL[dt], got, ref)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_raw_gain_decode_step(dt):
    d, T0, H = 64, 40, 4
    w = get_workload("tiny_t256_d32").resized(name=f"raw_dec_{dt}", B=1, H=H, T=T0 + 1, d=d,
                                              dtype=dt, lambda0=2.0)
    q, k, v, u = _rounded(w, make_inputs(w))
    pre = oracle_forward(q[:, :T0], k[:, :T0], v[:, :T0], u[:, :T0], w.lambda0, eps=w.eps,
                         gain="raw", return_n=True)
    S0, A0, n0 = (x.astype(np.float32) for x in pre[1:])
    ref = oracle_forward(q[:, T0:], k[:, T0:], v[:, T0:], u[:, T0:], w.lambda0, eps=w.eps,
                         gain="raw", state=(S0, A0, n0), return_n=True)
    dev = [_dev(x[:, T0:], w, (1, H, 1, d)) for x in (q, k, v, u)]
    _say(f"[case] raw gain decode step {dt}")
    out, S, A, n = vla.forward_state(*dev, 0.0, S0=torch.from_numpy(S0).view(1, H, d, d).cuda(),
                                     A0=torch.from_numpy(A0).view(1, H, d, d).cuda(),
                                     n0=torch.from_numpy(n0).view(1, H, d).cuda(), eps=w.eps,
                                     gain="raw")  # auto: decode
    torch.cuda.synchronize()
    got = (_np(out).reshape(H, 1, d), _np(S).reshape(H, d, d), _np(A).reshape(H, d, d),
           _np(n).reshape(H, d))
    _compare(f"raw gain decode {dt}", TOL[dt], got, ref)


@pytest.mark.parametrize("gain", ["unit", "raw"])
def test_transition_product_from_identity_state(gain):
    """S_0 = I and v = 0 give S_T = prod_t (I - khat_t g_t^T), matched against the oracle."""
    d, T, H, lam = 32, 25, 4, 0.25
    w = get_workload("tiny_t256_d32").resized(name=f"jac_{gain}", B=1, H=H, T=T, d=d, dtype="f32",
                                              lambda0=lam)
    q, k, v, u = make_inputs(w)
    v = np.zeros_like(v)
    S0 = np.broadcast_to(np.eye(d, dtype=np.float32), (H, d, d)).copy()
    A0 = np.broadcast_to(np.eye(d, dtype=np.float32) / np.float32(lam), (H, d, d)).copy()
    n0 = np.zeros((H, d), dtype=np.float32)
    ref = oracle_forward(q, k, v, u, lam, eps=w.eps, gain=gain, state=(S0, A0, n0), return_n=True)
    dev = [_dev(x, w, (1, H, T, d)) for x in (q, k, v, u)]
    out, S, A, n = vla.forward_state(*dev, lam, S0=torch.from_numpy(S0).view(1, H, d, d).cuda(),
                                     eps=w.eps, gain=gain, path="seq")
    torch.cuda.synchronize()
    got = (_np(out).reshape(H, T, d), _np(S).reshape(H, d, d), _np(A).reshape(H, d, d),
           _np(n).reshape(H, d))
    _compare(f"transition product {gain}", TOL["f32"], got, ref)
    norms = [np.linalg.norm(x, 2) for x in got[1]]
    _say(f"[info] ||prod J||_2 after {T} tokens, lambda0={lam}, {gain} gain: max {max(norms):.3e}")
