"""Parity of vla_backward against the fp64 autograd oracle (GPU only).

The oracle (oracle/vla_grad.py) is pinned to finite differences of the numpy forward on the
CPU.  Here every gradient (dq, dk, dv, du and dlambda0) of the loss <d_out, out> +
<dS_T, S_T> + <dA_T, A_T> + <dn_T, n_T> with random cotangents is compared by relative L2:
< 1e-4 for fp32 inputs, < 1e-2 for bf16 inputs (the oracle sees the bf16-rounded inputs and
cotangent).  Lengths cross the 32-token state checkpoints and end mid-interval.
"""

import sys

import numpy as np
import pytest
import torch

from rls_associative_memory_amd import vla
from rls_associative_memory_amd.inputs import get_workload, make_inputs, torch_dtype

from .parity import TOL, rel_l2
from oracle import vla_grad

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _run(d, dt, T, H=2, lam=0.8, with_state=True, seed=5, path="auto"):
    w = get_workload("tiny_t256_d32").resized(name=f"bw_{d}_{dt}_{T}", B=1, H=H, T=T, d=d,
                                              dtype=dt, lambda0=lam)
    q, k, v, u = make_inputs(w)
    r = np.random.default_rng(seed)
    dout = r.standard_normal(q.shape).astype(np.float32)
    dS = r.standard_normal((H, d, d)).astype(np.float32) if with_state else None
    dA = r.standard_normal((H, d, d)).astype(np.float32) if with_state else None
    dn = r.standard_normal((H, d)).astype(np.float32) if with_state else None
    dev = [torch.from_numpy(np.ascontiguousarray(x)).view(1, H, T, d).to(torch_dtype(w)).cuda()
           for x in (q, k, v, u, dout)]
    seen = [x.float().cpu().numpy().reshape(H, T, d).astype(np.float64) for x in dev]
    _say(f"[case] backward d={d} {dt} T={T} state cotangents={with_state} path={path}")
    tens = lambda x, shp: torch.from_numpy(x).view(shp).cuda() if x is not None else None
    got = vla.backward(*dev[:4], lam, dev[4], dS_T=tens(dS, (1, H, d, d)), dA_T=tens(dA, (1, H, d, d)),
                       dn_T=tens(dn, (1, H, d)), eps=w.eps, path=path)
    torch.cuda.synchronize()
    ref = vla_grad(*seen[:4], lam, seen[4], dS, dA, dn, eps=w.eps)
    tol = TOL[dt]
    names = ("dq", "dk", "dv", "du")
    errs = {n: rel_l2(g.cpu().numpy().reshape(H, T, d), rf) for n, g, rf in zip(names, got[:4], ref[:4])}
    errs["dlambda0"] = rel_l2(got[4].cpu().numpy().reshape(H), ref[4])
    _say(f"[parity] backward d={d} {dt} T={T}: " + " ".join(f"{n}={e:.3e}" for n, e in errs.items())
         + f" (tol {tol:g})")
    for n, e in errs.items():
        assert e < tol, f"{n} rel L2 {e:.3e} >= {tol:g}"


@pytest.mark.parametrize("d", [32, 64, 96, 128])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_backward_matches_oracle(d, dt):
    _run(d, dt, T=70)


@pytest.mark.parametrize("T", [1, 32, 33])
def test_backward_edge_lengths(T):
    _run(64, "f32", T=T)


# Time-segment parallel backward on shapes that split into several segments (64-token segments
# for fp32 inputs, 256-token ones for bf16), including a last segment of a single token.
@pytest.mark.parametrize("d,dt,T", [(64, "f32", 300), (32, "f32", 129), (96, "f32", 257),
                                    (64, "bf16", 1100), (128, "bf16", 600), (96, "bf16", 513),
                                    (32, "bf16", 777)])
def test_backward_segments_match_oracle(d, dt, T):
    _run(d, dt, T, path="chunk")


def test_backward_segments_without_state_cotangents():
    _run(64, "f32", T=200, with_state=False, lam=0.5, path="chunk")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_backward_few_long_streams(dt):
    """Two streams of 4096 tokens at d = 96 (64 segments of 64 tokens for fp32 inputs, 16 of
    256 for bf16), on the path the library picks for them (time segments), against the fp64
    oracle; the gradients of the token-by-token path beside them.  Bars as for the full
    workloads: the larger of the forward's bar and four times the deviation of the same
    steps in plain fp32 (dlambda0, a closed form, at the bar itself)."""
    H, T, d, lam = 2, 4096, 96, 0.8
    w = get_workload("tiny_t256_d32").resized(name=f"bw_long_{dt}", B=1, H=H, T=T, d=d, dtype=dt,
                                              lambda0=lam)
    q, k, v, u = make_inputs(w)
    r = np.random.default_rng(17)
    dout = r.standard_normal(q.shape).astype(np.float32)
    dS = r.standard_normal((H, d, d)).astype(np.float32)
    dA = r.standard_normal((H, d, d)).astype(np.float32)
    dn = r.standard_normal((H, d)).astype(np.float32)
    dev = [torch.from_numpy(np.ascontiguousarray(x)).view(1, H, T, d).to(torch_dtype(w)).cuda()
           for x in (q, k, v, u, dout)]
    seen = [x.float().cpu().numpy().reshape(H, T, d) for x in dev]
    cots = dict(dS_T=torch.from_numpy(dS).view(1, H, d, d).cuda(), dA_T=torch.from_numpy(dA).view(1, H, d, d).cuda(),
                dn_T=torch.from_numpy(dn).view(1, H, d).cuda())
    assert vla.backward_workspace_size((1, H, T, d), torch_dtype(w)) == \
        vla.backward_workspace_size((1, H, T, d), torch_dtype(w), path="chunk")
    _say(f"[case] backward few long streams {dt}: {H} x {T} tokens, d = {d}")
    got = vla.backward(*dev[:4], lam, dev[4], eps=w.eps, **cots)
    seq = vla.backward(*dev[:4], lam, dev[4], eps=w.eps, path="seq", **cots)
    torch.cuda.synchronize()
    ref = vla_grad(*(x.astype(np.float64) for x in seen[:4]), lam, seen[4].astype(np.float64),
                   dS.astype(np.float64), dA.astype(np.float64), dn.astype(np.float64), eps=w.eps)
    ref32 = vla_grad(*seen[:4], lam, seen[4], dS, dA, dn, eps=w.eps, dtype=torch.float32)
    tol = TOL[dt]
    names = ("dq", "dk", "dv", "du")
    bars = {n: max(tol, 4.0 * rel_l2(r32, rf)) for n, r32, rf in zip(names, ref32[:4], ref[:4])}
    bars["dlambda0"] = tol
    for label, res in (("segments", got), ("token by token", seq)):
        errs = {n: rel_l2(g.cpu().numpy().reshape(H, T, d), rf) for n, g, rf in zip(names, res[:4], ref[:4])}
        errs["dlambda0"] = rel_l2(res[4].cpu().numpy().reshape(H), ref[4])
        _say(f"[parity] backward {label} {dt}: " + " ".join(f"{n}={e:.3e} (bar {bars[n]:.1e})" for n, e in errs.items()))
        for n, e in errs.items():
            assert e < bars[n], f"{label}: {n} rel L2 {e:.3e} >= {bars[n]:.3e}"


def test_backward_without_state_cotangents_and_long():
    _run(64, "f32", T=300, with_state=False, lam=0.5)


@pytest.mark.parametrize("name,sample,path", [("mqar_t512_d32", (0, 77, 255), "auto"),
                                              ("mqar_t512_d32", (0, 77, 255), "seq"),
                                              ("iid_t4096_d64", (5,), "auto")])
def test_backward_full_workload_sampled_streams(name, sample, path):
    """Every stream of a full-size workload in one call (the launch bench.py times: AUTO, time
    segments on both workloads); the gradients of sampled streams against the oracle, and the
    recall workload with one segment per stream as well.  Cotangents are seeded per stream, so a
    sampled stream's cotangents are regenerated on the host without the others."""
    from rls_associative_memory_amd.inputs import make_inputs, upload_inputs
    w = get_workload(name)
    N, T, d = w.streams, w.T, w.d
    dt = torch_dtype(w)
    dev = upload_inputs(w, "cuda")

    def cot(s):
        r = np.random.default_rng([99, s])
        return (r.standard_normal((T, d)).astype(np.float32), r.standard_normal((d, d)).astype(np.float32),
                r.standard_normal((d, d)).astype(np.float32), r.standard_normal(d).astype(np.float32))

    host = [cot(s) for s in range(N)]
    dout = torch.from_numpy(np.stack([h[0] for h in host])).to(dt).view(w.B, w.H, T, d).cuda()
    dS = torch.from_numpy(np.stack([h[1] for h in host])).view(w.B, w.H, d, d).cuda()
    dA = torch.from_numpy(np.stack([h[2] for h in host])).view(w.B, w.H, d, d).cuda()
    dn = torch.from_numpy(np.stack([h[3] for h in host])).view(w.B, w.H, d).cuda()
    _say(f"[case] backward full {name}: {N} streams x {T} tokens, sampled {sample}, path {path}")
    got = vla.backward(*dev, w.lambda0, dout, dS_T=dS, dA_T=dA, dn_T=dn, eps=w.eps, path=path)
    torch.cuda.synchronize()
    q, k, v, u = make_inputs(w, streams=sample)
    douts = dout.float().view(N, T, d)[list(sample)].cpu().numpy().astype(np.float64)
    idx = list(sample)
    ref = vla_grad(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), u.astype(np.float64),
                   w.lambda0, douts, np.stack([host[s][1] for s in idx]).astype(np.float64),
                   np.stack([host[s][2] for s in idx]).astype(np.float64),
                   np.stack([host[s][3] for s in idx]).astype(np.float64), eps=w.eps)
    tol = TOL[w.dtype]
    names = ("dq", "dk", "dv", "du")
    errs = {n: rel_l2(g.view(N, T, d)[idx].cpu().numpy(), rf) for n, g, rf in zip(names, got[:4], ref[:4])}
    errs["dlambda0"] = rel_l2(got[4].view(N)[idx].cpu().numpy(), ref[4])
    # Where u_t = k_t (the recall layout) du is ill-conditioned: the same steps in plain fp32
    # stray from the fp64 gradients by about 4e-4.  dq, dk, dv, du are held to the larger of
    # the bar and four times that fp32 deviation; dlambda0 (closed form) to the bar itself.
    ref32 = vla_grad(q, k, v, u, w.lambda0, douts, np.stack([host[s][1] for s in idx]),
                     np.stack([host[s][2] for s in idx]), np.stack([host[s][3] for s in idx]),
                     eps=w.eps, dtype=torch.float32)
    bars = {n: max(tol, 4.0 * rel_l2(r32, rf)) for n, r32, rf in zip(names, ref32[:4], ref[:4])}
    bars["dlambda0"] = tol
    _say(f"[parity] backward full {name} {path}: " + " ".join(f"{n}={e:.3e} (bar {bars[n]:.1e})" for n, e in errs.items()))
    for n, e in errs.items():
        assert e < bars[n], f"{n} rel L2 {e:.3e} >= {bars[n]:.3e}"


# Time segments on the method's edge cases: u = 0 (the delta rule, A stays I / lambda0) and
# u = k with a small lambda0 (ill-conditioned segment starts), and d = 128 with fp32 inputs.
# Bars as for the long streams: the larger of the forward's bar and four times the deviation
# of the same steps in plain fp32 for dq, dk, dv, du; dlambda0 (a closed form) at the bar.
BW_EDGE = [("u0", "f32", 64, 300, 0.7), ("u0", "bf16", 96, 600, 0.7),
           ("uk", "f32", 32, 300, 0.05), ("uk", "bf16", 96, 1100, 0.05),
           ("iid", "f32", 128, 200, 0.9)]


@pytest.mark.parametrize("kind,dt,d,T,lam", BW_EDGE)
def test_backward_segments_edge_cases(kind, dt, d, T, lam):
    H = 2
    w = get_workload("tiny_t256_d32").resized(name=f"bwe_{kind}_{dt}_{d}_{T}", B=1, H=H, T=T, d=d,
                                              dtype=dt, lambda0=lam)
    q, k, v, u = make_inputs(w)
    if kind == "u0":
        u = np.zeros_like(u)
    elif kind == "uk":
        u = k.copy()
    r = np.random.default_rng([23, d, T])
    dout = r.standard_normal(q.shape).astype(np.float32)
    dS = r.standard_normal((H, d, d)).astype(np.float32)
    dA = r.standard_normal((H, d, d)).astype(np.float32)
    dn = r.standard_normal((H, d)).astype(np.float32)
    dev = [torch.from_numpy(np.ascontiguousarray(x)).view(1, H, T, d).to(torch_dtype(w)).cuda()
           for x in (q, k, v, u, dout)]
    seen = [x.float().cpu().numpy().reshape(H, T, d) for x in dev]
    _say(f"[case] backward time segments {kind} {dt} d={d} T={T} lambda0={lam}")
    got = vla.backward(*dev[:4], lam, dev[4], dS_T=torch.from_numpy(dS).view(1, H, d, d).cuda(),
                       dA_T=torch.from_numpy(dA).view(1, H, d, d).cuda(),
                       dn_T=torch.from_numpy(dn).view(1, H, d).cuda(), eps=w.eps, path="chunk")
    torch.cuda.synchronize()
    ref = vla_grad(*(x.astype(np.float64) for x in seen[:4]), lam, seen[4].astype(np.float64),
                   dS.astype(np.float64), dA.astype(np.float64), dn.astype(np.float64), eps=w.eps)
    ref32 = vla_grad(*seen[:4], lam, seen[4], dS, dA, dn, eps=w.eps, dtype=torch.float32)
    tol = TOL[dt]
    names = ("dq", "dk", "dv", "du")
    bars = {n: max(tol, 4.0 * rel_l2(r32, rf)) for n, r32, rf in zip(names, ref32[:4], ref[:4])}
    bars["dlambda0"] = tol
    errs = {n: rel_l2(g.cpu().numpy().reshape(H, T, d), rf) for n, g, rf in zip(names, got[:4], ref[:4])}
    errs["dlambda0"] = rel_l2(got[4].cpu().numpy().reshape(H), ref[4])
    _say(f"[parity] backward time segments {kind} {dt} d={d}: " +
         " ".join(f"{n}={e:.3e} (bar {bars[n]:.1e})" for n, e in errs.items()))
    for n, e in errs.items():
        assert e < bars[n], f"{n} rel L2 {e:.3e} >= {bars[n]:.3e}"
