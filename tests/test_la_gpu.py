"""Parity of the linear-attention baseline (vla_linear_attention) against its fp64 oracle
(GPU only).

Relative L2 per tensor (out, S_T, n_T) on identically rounded inputs, bars as for the VLA
path: 1e-4 for fp32 inputs, 1e-2 for bf16 inputs.  The shapes cover one partial chunk,
exactly one chunk, ragged tails, one chunk per segment and several chunks per segment (the
segment prefix), every head size, and a long case whose every stream the oracle runs in full.
"""

import sys

import numpy as np
import pytest
import torch

from rls_associative_memory_amd import vla
from rls_associative_memory_amd.inputs import get_workload, make_inputs, torch_dtype

from .parity import TOL, rel_l2
from oracle import la_forward

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _run_case(B, H, T, d, dt, seed_name="tiny_t256_d32"):
    w = get_workload(seed_name).resized(name=f"la_b{B}h{H}t{T}d{d}_{dt}", B=B, H=H, T=T, d=d, dtype=dt)
    q, k, v, _ = make_inputs(w)
    dev = [torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).view(B, H, T, d)
           .to(torch_dtype(w)).cuda() for x in (q, k, v)]
    rounded = [_np(x).reshape(B * H, T, d) for x in dev]  # the values the kernels see
    _say(f"[case] linear attention B={B} H={H} T={T} d={d} {dt} "
         f"workspace={vla.la_workspace_size((B, H, T, d), dev[0].dtype)} B")
    out, S, n = vla.linear_attention(*dev, eps=w.eps)
    torch.cuda.synchronize()
    ro, rS, rn = la_forward(*rounded, eps=w.eps)
    got = {"out": _np(out).reshape(B * H, T, d), "S": _np(S).reshape(B * H, d, d),
           "n": _np(n).reshape(B * H, d)}
    ref = {"out": ro, "S": rS, "n": rn}
    tol = TOL[dt]
    worst = {key: max(rel_l2(got[key][s], ref[key][s]) for s in range(B * H)) for key in got}
    _say(f"[parity] la B={B} H={H} T={T} d={d} {dt}: worst per-stream "
         + " ".join(f"{key}={e:.3e}" for key, e in worst.items()) + f" (tol {tol:g})")
    for key, e in worst.items():
        assert e < tol, f"{key} rel L2 {e:.3e} >= {tol:g}"


CASES = [(1, 2, T, d, dt) for d in (32, 64, 96, 128) for dt in ("f32", "bf16") for T in (300,)]
CASES += [(1, 1, T, 64, "f32") for T in (1, 5, 64, 65, 128)]
CASES += [(4, 16, 1100, d, dt) for d in (32, 128) for dt in ("f32", "bf16")]  # 3 chunks per segment


@pytest.mark.parametrize("B,H,T,d,dt", CASES)
def test_linear_attention_matches_oracle(B, H, T, d, dt):
    _run_case(B, H, T, d, dt)


def test_linear_attention_long_streams():
    """32 streams of 16384 tokens, d = 96, bf16 (the shape of the long VLA workload, shorter):
    16 segments of 16 chunks each; the oracle runs every stream in full."""
    _run_case(1, 32, 16384, 96, "bf16")


def test_linear_attention_deterministic():
    B, H, T, d = 1, 4, 2000, 64
    w = get_workload("tiny_t256_d32").resized(name="la_det", B=B, H=H, T=T, d=d, dtype="bf16")
    dev = [torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).view(B, H, T, d)
           .to(torch.bfloat16).cuda() for x in make_inputs(w)[:3]]
    a = vla.linear_attention(*dev)
    b = vla.linear_attention(*dev)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_linear_attention_full_long_workload_sampled():
    """The 131072-token workload (32 streams, d = 96, bf16) at full size in the launch
    configuration bench.py times: stream 0 checked in full against the oracle (out, S_T, n_T),
    the first 2048 tokens of streams 1 and 31 (causal prefix)."""
    from rls_associative_memory_amd.inputs import make_stream, upload_inputs
    w = get_workload("long_t131072_d96")
    q, k, v, _ = upload_inputs(w, "cuda")
    _say(f"[case] linear attention full long workload {w.B}x{w.H}x{w.T}x{w.d}")
    out, S, n = vla.linear_attention(q, k, v, eps=w.eps)
    torch.cuda.synchronize()
    o = out.view(-1, w.T, w.d)
    tol = TOL[w.dtype]
    for s, ntok in ((0, w.T), (1, 2048), (31, 2048)):
        qs, ks, vs, _ = (torch.from_numpy(x[:ntok]).to(torch.bfloat16).double().numpy()
                         for x in make_stream(w, s))
        ro, rS, rn = la_forward(qs, ks, vs, eps=w.eps)
        errs = {"out": rel_l2(_np(o[s, :ntok]), ro)}
        if ntok == w.T:
            errs["S"] = rel_l2(_np(S.view(-1, w.d, w.d)[s]), rS)
            errs["n"] = rel_l2(_np(n.view(-1, w.d)[s]), rn)
        _say(f"[parity] la long stream {s} ({ntok} tokens): "
             + " ".join(f"{key}={e:.3e}" for key, e in errs.items()) + f" (tol {tol:g})")
        for key, e in errs.items():
            assert e < tol, f"stream {s} {key} rel L2 {e:.3e} >= {tol:g}"
