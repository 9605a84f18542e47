"""Parity of the HIP path against the fp64 oracle (GPU only).

Every comparison is the relative L2 error ||x_gpu - x_ref|| / ||x_ref|| per tensor (out,
and S_T, A_T when requested) on identically rounded inputs; the bar is 1e-4 for fp32
inputs and 1e-2 for bf16 inputs.  Small shapes are checked on every stream; the long
workloads are run at full size and checked on sampled streams (streams are independent,
so a sampled stream's oracle needs only that stream's inputs).
"""

import sys

import numpy as np
import pytest
import torch

from rls_associative_memory_amd import vla
from rls_associative_memory_amd.inputs import get_workload, make_inputs, upload_inputs

from .parity import TOL, oracle_streams, rel_l2
from oracle import vla_forward as oracle_forward

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _to64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _check(w, streams, gpu_out, gpu_S, gpu_A, refs, label):
    tol = TOL[w.dtype]
    worst = {"out": 0.0, "S": 0.0, "A": 0.0}
    o = _to64(gpu_out).reshape(-1, w.T, w.d)
    S = _to64(gpu_S).reshape(-1, w.d, w.d) if gpu_S is not None else None
    A = _to64(gpu_A).reshape(-1, w.d, w.d) if gpu_A is not None else None
    for slot, (s, (ro, rS, rA)) in enumerate(zip(streams, refs)):
        worst["out"] = max(worst["out"], rel_l2(o[s], ro))
        if S is not None:
            worst["S"] = max(worst["S"], rel_l2(S[s], rS))
        if A is not None:
            worst["A"] = max(worst["A"], rel_l2(A[s], rA))
    _say(f"[parity] {label}: worst per-stream rel L2 out={worst['out']:.3e} "
         f"S={worst['S']:.3e} A={worst['A']:.3e} (tol {tol:g})")
    for key, val in worst.items():
        assert val < tol, f"{label}: {key} rel L2 {val:.3e} >= {tol:g}"


def _run(w, path, streams=None, chunk=0):
    q, k, v, u = upload_inputs(w, "cuda", streams=streams)
    out, S, A = vla.forward(q, k, v, u, w.lambda0, eps=w.eps, path=path, chunk=chunk,
                            return_state=True)
    torch.cuda.synchronize()
    return out, S, A


SMALL = [
    (d, dt, T)
    for d in (32, 64, 96, 128)
    for dt in ("f32", "bf16")
    for T in (1, 5, 37, 130)
]


@pytest.mark.parametrize("d,dt,T", SMALL)
def test_seq_small_shapes(d, dt, T):
    w = get_workload("tiny_t256_d32").resized(name=f"small_d{d}_{dt}_T{T}", B=1, H=3, T=T,
                                              d=d, dtype=dt, lambda0=0.7)
    _say(f"[case] seq small d={d} dtype={dt} T={T}")
    out, S, A = _run(w, "seq")
    q, k, v, u = make_inputs(w)
    refs = [oracle_forward(q[s], k[s], v[s], u[s], w.lambda0, eps=w.eps) for s in range(3)]
    _check(w, range(3), out, S, A, refs, f"seq d={d} {dt} T={T}")


@pytest.mark.parametrize("name", ["tiny_t256_d32", "mqar_t512_d32", "iid_t4096_d64"])
def test_seq_workloads_all_streams(name):
    w = get_workload(name)
    _say(f"[case] seq workload {name} (all streams)")
    out, S, A = _run(w, "seq")
    q, k, v, u = make_inputs(w)
    ro, rS, rA = oracle_forward(q, k, v, u, w.lambda0, eps=w.eps)
    refs = [(ro[s], rS[s], rA[s]) for s in range(w.streams)]
    _check(w, range(w.streams), out, S, A, refs, f"seq {name}")


@pytest.mark.parametrize("name,path", [("crossover_t43008_d128", "seq"),
                                       ("long_t131072_d96", "seq")])
def test_long_workloads_sampled_streams(name, path):
    w = get_workload(name)
    sample = [0, w.streams - 1]
    _say(f"[case] {path} workload {name} full size, sampled streams {sample}")
    out, S, A = _run(w, path)
    refs = oracle_streams(w, sample)
    o = out.view(-1, w.T, w.d)
    _check(w, range(len(sample)), o[sample], S.view(-1, w.d, w.d)[sample],
           A.view(-1, w.d, w.d)[sample], refs, f"{path} {name} sampled")


def test_zero_key_and_zero_u_tokens():
    w = get_workload("tiny_t256_d32").resized(name="zero_key", B=1, H=2, T=40, d=64,
                                              dtype="f32")
    q, k, v, u = make_inputs(w)
    k[:, 7] = 0.0
    u[:, 11] = 0.0
    k[:, 20] = 0.0
    u[:, 20] = 0.0
    dev = [torch.from_numpy(x).view(1, 2, w.T, w.d).cuda() for x in (q, k, v, u)]
    out, S, A = vla.forward(*dev, w.lambda0, eps=w.eps, path="seq", return_state=True)
    torch.cuda.synchronize()
    refs = [oracle_forward(q[s], k[s], v[s], u[s], w.lambda0, eps=w.eps) for s in range(2)]
    _check(w, range(2), out, S, A, refs, "zero key / zero u")


def test_deterministic_and_state_optional():
    w = get_workload("iid_t4096_d64").resized(name="det", B=2, H=2, T=300)
    q, k, v, u = upload_inputs(w, "cuda")
    o1, S1, A1 = vla.forward(q, k, v, u, w.lambda0, path="seq", return_state=True)
    o2, S2, A2 = vla.forward(q, k, v, u, w.lambda0, path="seq", return_state=True)
    o3 = vla.forward(q, k, v, u, w.lambda0, path="seq")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2) and torch.equal(A1, A2)
    assert torch.equal(o1, o3)
    assert torch.equal(A1, A1.transpose(-1, -2)), "A_T must be exactly symmetric"


def test_auto_path_runs_and_matches():
    w = get_workload("mqar_t512_d32").resized(name="auto", B=4, H=2, T=64)
    q, k, v, u = upload_inputs(w, "cuda")
    o_auto = vla.forward(q, k, v, u, w.lambda0)
    o_seq = vla.forward(q, k, v, u, w.lambda0, path="seq")
    torch.cuda.synchronize()
    if vla.resolve_path(tuple(q.shape), q.dtype) == "seq":
        assert torch.equal(o_auto, o_seq)


# ---------------------------------------------------------------------------------------
# Chunked, time-segment-parallel path
# ---------------------------------------------------------------------------------------

CHUNK_SMALL = [
    (d, dt, T, C)
    for d in (32, 64, 96, 128)
    for dt in ("f32", "bf16")
    for T in (1, 37, 300, 700)
    for C in (16, 32, 64)
    if not (d == 128 and C == 64)
]


@pytest.mark.parametrize("d,dt,T,C", CHUNK_SMALL)
def test_chunk_small_shapes(d, dt, T, C):
    w = get_workload("tiny_t256_d32").resized(name=f"chunk_d{d}_{dt}_T{T}_C{C}", B=1, H=3,
                                              T=T, d=d, dtype=dt, lambda0=0.7)
    _say(f"[case] chunk small d={d} dtype={dt} T={T} C={C}")
    out, S, A = _run(w, "chunk", chunk=C)
    q, k, v, u = make_inputs(w)
    refs = [oracle_forward(q[s], k[s], v[s], u[s], w.lambda0, eps=w.eps) for s in range(3)]
    _check(w, range(3), out, S, A, refs, f"chunk d={d} {dt} T={T} C={C}")


@pytest.mark.parametrize("name", ["mqar_t512_d32", "iid_t4096_d64"])
def test_chunk_workloads_all_streams(name):
    w = get_workload(name)
    _say(f"[case] chunk workload {name} (all streams)")
    out, S, A = _run(w, "chunk")
    q, k, v, u = make_inputs(w)
    ro, rS, rA = oracle_forward(q, k, v, u, w.lambda0, eps=w.eps)
    refs = [(ro[s], rS[s], rA[s]) for s in range(w.streams)]
    _check(w, range(w.streams), out, S, A, refs, f"chunk {name}")


@pytest.mark.parametrize("name", ["crossover_t43008_d128", "long_t131072_d96"])
def test_chunk_long_workloads_sampled_streams(name):
    w = get_workload(name)
    sample = [0, w.streams - 1]
    _say(f"[case] chunk workload {name} full size, sampled streams {sample}")
    out, S, A = _run(w, "chunk", chunk=w.chunk)
    refs = oracle_streams(w, sample)
    _check(w, range(len(sample)), out.view(-1, w.T, w.d)[sample],
           S.view(-1, w.d, w.d)[sample], A.view(-1, w.d, w.d)[sample], refs,
           f"chunk {name} sampled")


def test_chunk_deterministic_and_workspace():
    w = get_workload("long_t131072_d96").resized(name="det_chunk", B=1, H=3, T=5000)
    q, k, v, u = upload_inputs(w, "cuda")
    n = vla.workspace_size(tuple(q.shape), q.dtype, path="chunk", chunk=64)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    o1, S1, A1 = vla.forward(q, k, v, u, w.lambda0, path="chunk", chunk=64, return_state=True,
                             workspace=ws)
    o2, S2, A2 = vla.forward(q, k, v, u, w.lambda0, path="chunk", chunk=64, return_state=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2) and torch.equal(A1, A2)
    small = torch.empty(max(n // 2, 16), dtype=torch.uint8, device="cuda")
    with pytest.raises(vla.VlaError):
        vla.forward(q, k, v, u, w.lambda0, path="chunk", chunk=64, workspace=small)


def test_chunk_zero_key_tokens():
    w = get_workload("tiny_t256_d32").resized(name="zero_key_chunk", B=1, H=2, T=600, d=64,
                                              dtype="f32")
    q, k, v, u = make_inputs(w)
    k[:, 7] = 0.0
    k[:, 300] = 0.0
    u[:, 11] = 0.0
    dev = [torch.from_numpy(x).view(1, 2, w.T, w.d).cuda() for x in (q, k, v, u)]
    out, S, A = vla.forward(*dev, w.lambda0, eps=w.eps, path="chunk", chunk=32, return_state=True)
    torch.cuda.synchronize()
    refs = [oracle_forward(q[s], k[s], v[s], u[s], w.lambda0, eps=w.eps) for s in range(2)]
    _check(w, range(2), out, S, A, refs, "chunk zero key / zero u")


@pytest.mark.parametrize("path,dt", [("chunk", "bf16"), ("chunk", "f32"), ("seq", "bf16")])
def test_forward_graph_replays_match_eager(path, dt):
    """A whole vla_forward call (every kernel of the path) captured in one HIP graph with a
    caller-owned workspace, replayed three times with eager work and synchronisations in
    between: every replay must equal the eager call bitwise."""
    w = get_workload("long_t131072_d96").resized(name=f"graph_{path}_{dt}", B=1, H=3, T=3000, dtype=dt)
    q, k, v, u = upload_inputs(w, "cuda")
    n = vla.workspace_size(tuple(q.shape), q.dtype, path=path, chunk=64)
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda") if n else None
    out = torch.empty_like(q)
    S = torch.empty((1, 3, w.d, w.d), dtype=torch.float32, device="cuda")
    A = torch.empty_like(S)

    def call():
        vla.forward(q, k, v, u, w.lambda0, path=path, chunk=64, out=out, S_final=S, A_final=A, workspace=ws)

    _say(f"[case] forward graph {path} {dt}: 3 x 3000 tokens, d = 96")
    call()
    torch.cuda.synchronize()
    ref = (out.clone(), S.clone(), A.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (out, S, A):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = all(torch.equal(a, b) for a, b in zip((out, S, A), ref))
        _say(f"[parity] forward graph {path} {dt} replay {rep}: bitwise equal to eager: {same}")
        assert same, f"replay {rep} differs from the eager call"
        _ = (torch.ones(4096, device="cuda") * 3.0).sum().item()  # eager work between replays
