"""Carried state (vla_forward_state): parity against the fp64 oracle continuing a stream,
and continuation identities on the device (GPU only).

A stream is run by the oracle over a prefix of tokens; the state it ends in (S, A, n,
rounded to fp32) is handed to the library, which continues over the next tokens.  The
oracle continues from the same fp32 values.  Bars as for vla_forward: relative L2 < 1e-4
(fp32 inputs), < 1e-2 (bf16 inputs) per tensor, here also for n_T.  On the device,
splitting a sequence into two calls (or into T = 1 decode steps) must give the single
call's result to the same bars.
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


def _dev(x, w, shape):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).view(shape).to(
        torch_dtype(w)).cuda()


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _case(d, dt, T0, T1, H=3):
    """Inputs rounded as the library sees them, the oracle state after T0 tokens (in fp32)
    and the oracle's continuation over the next T1 tokens from that state."""
    w = get_workload("tiny_t256_d32").resized(name=f"state_d{d}_{dt}", B=1, H=H, T=T0 + T1, d=d,
                                              dtype=dt, lambda0=0.8)
    q, k, v, u = make_inputs(w)
    if dt == "bf16":  # the oracle sees the bf16-rounded values
        q, k, v, u = (torch.from_numpy(x).to(torch.bfloat16).float().numpy() for x in (q, k, v, u))
    pre = oracle_forward(q[:, :T0], k[:, :T0], v[:, :T0], u[:, :T0], w.lambda0, eps=w.eps,
                         return_n=True)
    state = tuple(x.astype(np.float32) for x in pre[1:])  # S, A, n
    ref = oracle_forward(q[:, T0:], k[:, T0:], v[:, T0:], u[:, T0:], w.lambda0, eps=w.eps,
                         state=state, return_n=True)
    return w, (q, k, v, u), state, ref


def _compare(label, tol, got, ref):
    names = ("out", "S", "A", "n")
    worst = {n: rel_l2(g, r) for n, g, r in zip(names, got, ref)}
    _say(f"[parity] {label}: " + " ".join(f"{n}={e:.3e}" for n, e in worst.items()) + f" (tol {tol:g})")
    for n, e in worst.items():
        assert e < tol, f"{label}: {n} rel L2 {e:.3e} >= {tol:g}"


STATE_CASES = [(d, dt, path) for d in (32, 64, 96, 128) for dt in ("f32", "bf16")
               for path in ("seq", "chunk")]


@pytest.mark.parametrize("d,dt,path", STATE_CASES)
def test_state_continuation_matches_oracle(d, dt, path):
    T0, T1 = 150, 1100 if path == "chunk" else 300
    _say(f"[case] carried state d={d} {dt} path={path} T0={T0} T1={T1}")
    w, (q, k, v, u), (S0, A0, n0), ref = _case(d, dt, T0, T1)
    H = w.H
    shp = (1, H, T1, d)
    dq, dk, dv, du = (_dev(x[:, T0:], w, shp) for x in (q, k, v, u))
    S0d = torch.from_numpy(S0).view(1, H, d, d).cuda()
    A0d = torch.from_numpy(A0).view(1, H, d, d).cuda()
    n0d = torch.from_numpy(n0).view(1, H, d).cuda()
    chunk = 32 if d > 96 else 64
    out, S, A, n = vla.forward_state(dq, dk, dv, du, 0.0, S0=S0d, A0=A0d, n0=n0d, eps=w.eps,
                                     path=path, chunk=chunk if path == "chunk" else 0)
    torch.cuda.synchronize()
    got = (_np(out).reshape(H, T1, d), _np(S).reshape(H, d, d), _np(A).reshape(H, d, d),
           _np(n).reshape(H, d))
    _compare(f"state d={d} {dt} {path}", TOL[dt], got, ref)


# A chunked-path call of at least 2^20 tokens on two or more streams runs its streams as two
# groups, the second on a second HIP stream of the library, each with its own slices of the
# inputs, outputs, carried states and workspace.  An odd stream count gives groups of unequal
# size (here 2 and 3); every stream is checked on its own against the oracle.  The wide
# workloads (32 streams at d = 96 and d = 128) cover the two groups at full size.
@pytest.mark.timeout(600)
def test_state_continuation_two_stream_groups():
    d, H, T0, T1 = 32, 5, 100, 210000
    assert H * T1 >= 1 << 20
    _say(f"[case] carried state, two stream groups: {H} streams x {T1} tokens, d={d}, bf16")
    w, (q, k, v, u), (S0, A0, n0), ref = _case(d, "bf16", T0, T1, H=H)
    shp = (1, H, T1, d)
    dq, dk, dv, du = (_dev(x[:, T0:], w, shp) for x in (q, k, v, u))
    out, S, A, n = vla.forward_state(dq, dk, dv, du, 0.0, S0=torch.from_numpy(S0).view(1, H, d, d).cuda(),
                                     A0=torch.from_numpy(A0).view(1, H, d, d).cuda(),
                                     n0=torch.from_numpy(n0).view(1, H, d).cuda(), eps=w.eps,
                                     path="chunk", chunk=64)
    torch.cuda.synchronize()
    got = (_np(out).reshape(H, T1, d), _np(S).reshape(H, d, d), _np(A).reshape(H, d, d),
           _np(n).reshape(H, d))
    for s in range(H):
        _compare(f"two groups d={d} stream {s}", TOL["bf16"], tuple(g[s] for g in got),
                 tuple(r[s] for r in ref))


@pytest.mark.parametrize("path", ["seq", "chunk"])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_two_calls_equal_one_call(path, dt):
    d, T = 64, 1400
    split = 611
    w = get_workload("tiny_t256_d32").resized(name="split", B=1, H=2, T=T, d=d, dtype=dt,
                                              lambda0=0.6)
    _say(f"[case] two calls vs one: {dt} path={path} T={T} split={split}")
    q, k, v, u = make_inputs(w)
    full = [_dev(x, w, (1, 2, T, d)) for x in (q, k, v, u)]
    o1, S1, A1, n1 = vla.forward_state(*full, w.lambda0, eps=w.eps, path=path)
    a = [x[:, :, :split].contiguous() for x in full]
    b = [x[:, :, split:].contiguous() for x in full]
    oa, Sa, Aa, na = vla.forward_state(*a, w.lambda0, eps=w.eps, path=path)
    ob, Sb, Ab, nb = vla.forward_state(*b, w.lambda0, S0=Sa, A0=Aa, n0=na, eps=w.eps, path=path)
    torch.cuda.synchronize()
    got = (_np(torch.cat([oa, ob], dim=2)), _np(Sb), _np(Ab), _np(nb))
    ref = (_np(o1), _np(S1), _np(A1), _np(n1))
    _compare(f"two calls {dt} {path}", TOL[dt], got, ref)


def test_decode_steps_equal_one_call():
    d, T = 96, 24
    w = get_workload("tiny_t256_d32").resized(name="decode", B=1, H=4, T=T, d=d, dtype="bf16",
                                              lambda0=0.5)
    _say(f"[case] {T} decode steps (T = 1 calls) vs one call, d={d}")
    q, k, v, u = make_inputs(w)
    full = [_dev(x, w, (1, 4, T, d)) for x in (q, k, v, u)]
    o1, S1, A1, n1 = vla.forward_state(*full, w.lambda0, eps=w.eps, path="seq")
    S = A = n = None
    outs = []
    for t in range(T):
        step = [x[:, :, t:t + 1].contiguous() for x in full]
        o, S, A, n = vla.forward_state(*step, w.lambda0, S0=S, A0=A, n0=n, eps=w.eps, path="seq")
        outs.append(o)
    torch.cuda.synchronize()
    got = (_np(torch.cat(outs, dim=2)), _np(S), _np(A), _np(n))
    ref = (_np(o1), _np(S1), _np(A1), _np(n1))
    _compare("decode steps", TOL["bf16"], got, ref)


DECODE_CASES = [(d, dt) for d in (32, 64, 96, 128) for dt in ("f32", "bf16")]


@pytest.mark.parametrize("d,dt", DECODE_CASES)
def test_decode_kernel_matches_oracle(d, dt):
    """One token per stream on the decode path from an oracle state after 150 tokens."""
    T0, T1 = 150, 1
    _say(f"[case] decode kernel d={d} {dt}")
    w, (q, k, v, u), (S0, A0, n0), ref = _case(d, dt, T0, T1, H=5)
    H = w.H
    dq, dk, dv, du = (_dev(x[:, T0:], w, (1, H, 1, d)) for x in (q, k, v, u))
    out, S, A, n = vla.forward_state(dq, dk, dv, du, 0.0, S0=torch.from_numpy(S0).view(1, H, d, d).cuda(),
                                     A0=torch.from_numpy(A0).view(1, H, d, d).cuda(),
                                     n0=torch.from_numpy(n0).view(1, H, d).cuda(), eps=w.eps,
                                     path="decode")
    torch.cuda.synchronize()
    got = (_np(out).reshape(H, 1, d), _np(S).reshape(H, d, d), _np(A).reshape(H, d, d),
           _np(n).reshape(H, d))
    _compare(f"decode d={d} {dt}", TOL[dt], got, ref)
    Af = A.view(H, d, d)
    assert torch.equal(Af, Af.transpose(1, 2)), "decode kept A exactly symmetric"


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_decode_path_steps_equal_one_call(dt):
    d, T = 64, 40
    w = get_workload("tiny_t256_d32").resized(name="decode_steps", B=2, H=3, T=T, d=d, dtype=dt,
                                              lambda0=0.9)
    _say(f"[case] {T} decode-path steps vs one sequential call, {dt}")
    q, k, v, u = make_inputs(w)
    full = [_dev(x, w, (2, 3, T, d)) for x in (q, k, v, u)]
    o1, S1, A1, n1 = vla.forward_state(*full, w.lambda0, eps=w.eps, path="seq")
    S = A = n = None
    outs = []
    for t in range(T):
        step = [x[:, :, t:t + 1].contiguous() for x in full]
        o, S, A, n = vla.forward_state(*step, w.lambda0, S0=S, A0=A, n0=n, eps=w.eps)  # auto: decode
        outs.append(o)
    torch.cuda.synchronize()
    got = (_np(torch.cat(outs, dim=2)), _np(S), _np(A), _np(n))
    ref = (_np(o1), _np(S1), _np(A1), _np(n1))
    _compare(f"decode path steps {dt}", TOL[dt], got, ref)


def test_decode_zero_key_and_zero_gain():
    d = 32
    w = get_workload("tiny_t256_d32").resized(name="decode_zero", B=1, H=2, T=1, d=d, dtype="f32")
    q, k, v, u = make_inputs(w)
    k[0] = 0.0  # stream 0: zero key (no memory write, A still downdates)
    ref = oracle_forward(q, k, v, u, w.lambda0, eps=w.eps, return_n=True)
    dev = [_dev(x, w, (1, 2, 1, d)) for x in (q, k, v, u)]
    out, S, A, n = vla.forward_state(*dev, w.lambda0, eps=w.eps, path="decode")
    torch.cuda.synchronize()
    got = (_np(out).reshape(2, 1, d), _np(S).reshape(2, d, d), _np(A).reshape(2, d, d),
           _np(n).reshape(2, d))
    _compare("decode zero key", TOL["f32"], got, ref)


def test_default_state_equals_vla_forward():
    w = get_workload("tiny_t256_d32").resized(name="defaults", B=1, H=2, T=700, d=96, dtype="bf16")
    q, k, v, u = make_inputs(w)
    dev = [_dev(x, w, (1, 2, w.T, w.d)) for x in (q, k, v, u)]
    for path in ("seq", "chunk"):
        o1, S1, A1 = vla.forward(*dev, w.lambda0, eps=w.eps, path=path, return_state=True)
        o2, S2, A2, _ = vla.forward_state(*dev, w.lambda0, eps=w.eps, path=path)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(S1, S2) and torch.equal(A1, A2), path


def test_decode_kernel_many_streams_sampled():
    """2048 streams (the decode bench's --decode-batch 64 shape, d = 96, bf16) from a carried
    state: sampled streams checked against the oracle's single step."""
    d, H, B = 96, 32, 64
    w = get_workload("long_t131072_d96").resized(name="decode_many", B=B, H=H, T=2)
    q, k, v, u = make_inputs(w)
    q, k, v, u = (torch.from_numpy(x).to(torch.bfloat16).float().numpy() for x in (q, k, v, u))
    streams = B * H
    rng = np.random.default_rng(11)
    # a valid carried state per stream: the oracle's state after the first token
    pre = oracle_forward(q[:, :1], k[:, :1], v[:, :1], u[:, :1], w.lambda0, eps=w.eps, return_n=True)
    S0, A0, n0 = (x.astype(np.float32) for x in pre[1:])
    dev = [_dev(x[:, 1:], w, (B, H, 1, d)) for x in (q, k, v, u)]
    _say(f"[case] decode kernel {streams} streams d={d}")
    out, S, A, n = vla.forward_state(*dev, 0.0, S0=torch.from_numpy(S0).view(B, H, d, d).cuda(),
                                     A0=torch.from_numpy(A0).view(B, H, d, d).cuda(),
                                     n0=torch.from_numpy(n0).view(B, H, d).cuda(), eps=w.eps)
    torch.cuda.synchronize()
    pick = np.sort(rng.choice(streams, 16, replace=False))
    st = (S0[pick], A0[pick], n0[pick])
    ref = oracle_forward(q[pick, 1:], k[pick, 1:], v[pick, 1:], u[pick, 1:], w.lambda0, eps=w.eps,
                         state=st, return_n=True)
    got = (_np(out).reshape(streams, 1, d)[pick], _np(S).reshape(streams, d, d)[pick],
           _np(A).reshape(streams, d, d)[pick], _np(n).reshape(streams, d)[pick])
    _compare(f"decode {streams} streams (16 sampled)", TOL["bf16"], got, ref)


def test_decode_graph_replays_match_eager():
    """A block of T = 1 decode calls captured in one HIP graph (the library enqueues only
    kernels on the caller's stream, no allocation or memset), replayed three times with eager
    work and synchronisations in between; every replay must equal the eager calls bitwise."""
    d, nst = 96, 6
    w = get_workload("tiny_t256_d32").resized(name="decode_graph", B=2, H=4, T=nst, d=d, dtype="bf16",
                                              lambda0=0.5)
    q, k, v, u = make_inputs(w)
    full = [_dev(x, w, (2, 4, nst, d)) for x in (q, k, v, u)]
    steps = [[x[:, :, t:t + 1].contiguous() for x in full] for t in range(nst)]
    mat = (2, 4, d, d)
    # a carried start state from a 50-token forward (so A0 and S0 are not trivial)
    pre = get_workload("tiny_t256_d32").resized(name="decode_graph_pre", B=2, H=4, T=50, d=d, dtype="bf16",
                                                lambda0=0.5)
    pq = [_dev(x, pre, (2, 4, 50, d)) for x in make_inputs(pre)]
    _, S_init, A_init, n_init = vla.forward_state(*pq, pre.lambda0, eps=pre.eps, path="seq")
    st = [(torch.empty(mat, device="cuda"), torch.empty(mat, device="cuda"),
           torch.empty((2, 4, d), device="cuda")) for _ in range(2)]
    outs = [torch.empty_like(steps[0][0]) for _ in range(nst)]

    def reset():
        for dst, src in zip(st[0], (S_init, A_init, n_init)):
            dst.copy_(src)

    def run():
        for t in range(nst):
            S0, A0, n0 = st[t & 1]
            S1, A1, n1 = st[(t & 1) ^ 1]
            vla.forward_state(*steps[t], w.lambda0, S0=S0, A0=A0, n0=n0, eps=w.eps, path="decode",
                              out=outs[t], S_final=S1, A_final=A1, n_final=n1)

    _say("[case] decode graph: 6 T = 1 calls, 8 streams, d = 96, bf16; eager reference")
    reset()
    run()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs] + [x.clone() for x in st[0]]
    g = torch.cuda.CUDAGraph()
    reset()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.zero_()
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = outs + list(st[0])
        same = all(torch.equal(a, b) for a, b in zip(got, ref))
        _say(f"[parity] decode graph replay {rep}: bitwise equal to eager: {same}")
        assert same, f"replay {rep} differs from the eager calls"
        _ = (torch.ones(1024, device="cuda") * 2.0).sum().item()  # eager work between replays
