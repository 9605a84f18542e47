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


@pytest.mark.parametrize("T,C", [(37, 16), (700, 32), (1300, 64)])
def test_chunk_two_streams_per_workgroup(T, C):
    """bf16 inputs at d = 96 with an even number of streams run the A side and the final pass
    with the same segment of two streams in one workgroup; an odd number runs one stream per
    workgroup.  On 4 streams: parity of every stream against the oracle, and the first 3 streams
    bitwise equal to a 3-stream call on the same inputs (both calls have the same segments: at
    most 4 x 1300 tokens per call, far below 2048 segments of the shortest bf16 length, 256)."""
    w = get_workload("long_t131072_d96").resized(name=f"pair_T{T}_C{C}", B=1, H=4, T=T, lambda0=0.7)
    _say(f"[case] two streams per workgroup: 4 (and 3) x {T} tokens, d = 96, C = {C}")
    out4, S4, A4 = _run(w, "chunk", chunk=C)
    out3, S3, A3 = _run(w, "chunk", streams=range(3), chunk=C)
    q, k, v, u = make_inputs(w)
    refs = [oracle_forward(q[s], k[s], v[s], u[s], w.lambda0, eps=w.eps) for s in range(4)]
    _check(w, range(4), out4, S4, A4, refs, f"pair d=96 bf16 T={T} C={C}")
    same = [torch.equal(a.reshape(-1)[: b.numel()], b.reshape(-1))
            for a, b in ((out4, out3), (S4, S3), (A4, A3))]
    _say(f"[parity] pair T={T} C={C}: streams 0..2 of 4 bitwise equal to 3 streams: {same}")
    assert all(same)


@pytest.mark.parametrize("name", ["mqar_t512_d32", "iid_t4096_d64"])
def test_chunk_workloads_all_streams(name):
    w = get_workload(name)
    _say(f"[case] chunk workload {name} (all streams)")
    out, S, A = _run(w, "chunk")
    q, k, v, u = make_inputs(w)
    ro, rS, rA = oracle_forward(q, k, v, u, w.lambda0, eps=w.eps)
    refs = [(ro[s], rS[s], rA[s]) for s in range(w.streams)]
    _check(w, range(w.streams), out, S, A, refs, f"chunk {name}")


# Eight streams of the two long workloads, interior ones included (the oracle of each runs in
# a worker process).  Besides the whole-stream error, the output is checked block by block over
# 256-token blocks: every segment of the chunked path at these sizes (1024 and 2048 tokens)
# starts on a block boundary, so an error confined to segment starts (a wrong segment-start
# state) cannot hide in the average over a whole stream.
SAMPLE8 = [0, 5, 11, 16, 21, 26, 30, 31]
BLOCK = 256


def _block_errors(x, ref, block):
    """Relative L2 of x against ref over each block of `block` tokens (axis 0)."""
    n = (ref.shape[0] + block - 1) // block
    return np.array([rel_l2(x[i * block:(i + 1) * block], ref[i * block:(i + 1) * block])
                     for i in range(n)])


def _token_errors(x, ref):
    num = np.linalg.norm(x - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    return num / np.where(den > 0, den, 1.0)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["crossover_t43008_d128", "long_t131072_d96"])
def test_chunk_long_workloads_eight_streams(name):
    w = get_workload(name)
    _say(f"[case] chunk workload {name} full size, streams {SAMPLE8}, per-{BLOCK}-token blocks")
    out, S, A = _run(w, "chunk", chunk=w.chunk)
    tol = TOL[w.dtype]
    o = out.view(-1, w.T, w.d)[SAMPLE8]
    Sg = S.view(-1, w.d, w.d)[SAMPLE8]
    Ag = A.view(-1, w.d, w.d)[SAMPLE8]
    _say(f"[case] {name}: oracle on {len(SAMPLE8)} streams in worker processes")
    refs = oracle_streams(w, SAMPLE8)
    _check(w, range(len(SAMPLE8)), o, Sg, Ag, refs, f"chunk {name} eight streams")
    o64 = _to64(o)
    worst_block, worst_tok = 0.0, 0.0
    for slot, (s, (ro, _, _)) in enumerate(zip(SAMPLE8, refs)):
        be = _block_errors(o64[slot], ro, BLOCK)
        te = _token_errors(o64[slot], ro)
        _say(f"[parity] {name} stream {s}: worst {BLOCK}-token block rel L2 {be.max():.3e} "
             f"(block {int(be.argmax())}), worst token rel L2 {te.max():.3e} (token {int(te.argmax())})")
        worst_block = max(worst_block, float(be.max()))
        worst_tok = max(worst_tok, float(te.max()))
        assert be.max() < tol, f"{name} stream {s}: block {int(be.argmax())} rel L2 {be.max():.3e}"
    _say(f"[parity] {name}: worst block {worst_block:.3e}, worst token {worst_tok:.3e} (tol {tol:g})")


def test_tiny_workload_on_its_automatic_path():
    """The 256-token fp32 workload (one stream, lambda0 = 1, eps = 1e-6) at its exact
    settings, on the path the library picks for it (the chunked path, 64-token segments) and
    on the chunked path forced."""
    w = get_workload("tiny_t256_d32")
    assert vla.resolve_path((w.B, w.H, w.T, w.d), torch.float32) == "chunk"
    q, k, v, u = make_inputs(w)
    refs = [oracle_forward(q[0], k[0], v[0], u[0], w.lambda0, eps=w.eps)]
    for path in ("auto", "chunk"):
        _say(f"[case] tiny_t256_d32 path={path}")
        out, S, A = _run(w, path)
        _check(w, [0], out, S, A, refs, f"tiny_t256_d32 {path}")
        be = _block_errors(_to64(out).reshape(w.T, w.d), refs[0][0], 64)
        _say(f"[parity] tiny_t256_d32 {path}: per-segment rel L2 {np.array2string(be, precision=2)}")
        assert be.max() < TOL[w.dtype]


# Chunked-path cases at the method's edges, all streams against the oracle.
#   u = 0 over whole streams: the penalty never grows, A stays I / lambda0 (the delta rule);
#   u = k with lambda0 = 0.01: the segment-start inverse penalties lambda0 I + sum u u^T of
#     short first segments are badly conditioned (eigenvalues lambda0 beside ~ tokens);
#   more than 16 segments per stream: the multi-pass loops of the segment prefix scans.
# With u = k and a small lambda0 the recurrence itself is ill-conditioned in fp32: while fewer
# than d keys have been seen, A_t khat is a difference of two terms about 1 + ||k||^2 / lambda0
# times larger than itself, so any fp32 evaluation of the printed steps strays from the fp64
# oracle by ~1e-3.  The bar of each tensor is therefore the larger of the dtype's tolerance and
# four times the deviation of the oracle's own steps evaluated in plain fp32 on the same input
# (for every other case here that deviation is ~1e-6 and the bar is the tolerance itself).
EDGE = [
    ("u0", "f32", 64, 700, 0.7), ("u0", "bf16", 96, 1300, 0.7), ("u0", "bf16", 32, 900, 1.0),
    ("uk", "f32", 32, 400, 0.01), ("uk", "f32", 96, 400, 0.01),
    ("uk", "bf16", 32, 1100, 0.01), ("uk", "bf16", 96, 1100, 0.01),
    ("iid", "f32", 32, 1500, 0.7), ("iid", "bf16", 64, 4500, 0.7),
]


def _fp32_deviation(q, k, v, u, lam, eps, refs):
    """Largest rel L2 (over streams) of the oracle's steps in plain fp32 against fp64, per
    tensor (out, S_T, A_T)."""
    from oracle import vla_forward_torch
    t = [torch.tensor(np.asarray(x), dtype=torch.float32) for x in (q, k, v, u)]
    lamv = torch.full((t[0].shape[0],), float(lam), dtype=torch.float32)
    o32, S32, A32, _ = vla_forward_torch(*t, lamv, eps=eps)
    dev = {"out": 0.0, "S": 0.0, "A": 0.0}
    for s, (ro, rS, rA) in enumerate(refs):
        dev["out"] = max(dev["out"], rel_l2(o32[s].double().numpy(), ro))
        dev["S"] = max(dev["S"], rel_l2(S32[s].double().numpy(), rS))
        dev["A"] = max(dev["A"], rel_l2(A32[s].double().numpy(), rA))
    return dev


@pytest.mark.parametrize("kind,dt,d,T,lam", EDGE)
def test_chunk_edge_cases(kind, dt, d, T, lam):
    w = get_workload("tiny_t256_d32").resized(name=f"edge_{kind}_{dt}_d{d}_T{T}", B=1, H=3,
                                              T=T, d=d, dtype=dt, lambda0=lam)
    q, k, v, u = make_inputs(w)
    if kind == "u0":
        u = np.zeros_like(u)
    elif kind == "uk":
        u = k.copy()
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    dev = [torch.from_numpy(x).view(1, 3, T, d).to(tdt).cuda() for x in (q, k, v, u)]
    assert vla.resolve_path((1, 3, T, d), tdt, path="chunk") == "chunk"
    _say(f"[case] chunk edge {kind} {dt} d={d} T={T} lambda0={lam}")
    out, S, A = vla.forward(*dev, lam, eps=w.eps, path="chunk", return_state=True)
    torch.cuda.synchronize()
    refs = [oracle_forward(q[s], k[s], v[s], u[s], lam, eps=w.eps) for s in range(3)]
    tol = TOL[dt]
    f32dev = _fp32_deviation(q, k, v, u, lam, w.eps, refs)
    bars = {key: max(tol, 4.0 * val) for key, val in f32dev.items()}
    got = {"out": _to64(out).reshape(3, T, d), "S": _to64(S).reshape(3, d, d),
           "A": _to64(A).reshape(3, d, d)}
    idx = {"out": 0, "S": 1, "A": 2}
    errs = {key: max(rel_l2(got[key][s], refs[s][idx[key]]) for s in range(3)) for key in got}
    worst_blk = max(float(_block_errors(got["out"][s], refs[s][0], 64).max()) for s in range(3))
    _say(f"[parity] chunk edge {kind} {dt} d={d} T={T} lambda0={lam}: "
         + " ".join(f"{key}={errs[key]:.3e} (fp32 steps {f32dev[key]:.1e}, bar {bars[key]:.1e})" for key in errs)
         + f"; worst 64-token block of out {worst_blk:.3e}")
    for key in errs:
        assert errs[key] < bars[key], f"{key} rel L2 {errs[key]:.3e} >= {bars[key]:.3e}"
    assert worst_blk < bars["out"]


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


@pytest.mark.parametrize("d", [32, 96])
def test_two_stream_groups_equal_one_launch(d):
    """A chunked call of at least 2^20 tokens runs its streams as two groups on two HIP streams
    (here 2 and 3 of 5 streams); the same call captured in a HIP graph runs as one launch over
    all streams (the library does not split under capture).  The segment length is the whole
    call's in both, so the outputs must be bitwise equal."""
    T = 1 << 18
    w = get_workload("long_t131072_d96").resized(name=f"groups_d{d}", B=1, H=5, T=T, d=d)
    q, k, v, u = upload_inputs(w, "cuda")
    n = vla.workspace_size(tuple(q.shape), q.dtype, path="chunk", chunk=64)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    S = torch.empty((1, 5, d, d), dtype=torch.float32, device="cuda")
    A = torch.empty_like(S)

    def call():
        vla.forward(q, k, v, u, w.lambda0, path="chunk", chunk=64, out=out, S_final=S, A_final=A, workspace=ws)

    _say(f"[case] two stream groups vs one launch: 5 x {T} tokens, d = {d}")
    call()
    torch.cuda.synchronize()
    eager = (out.clone(), S.clone(), A.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for t in (out, S, A):
        t.zero_()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    same = [torch.equal(a, b) for a, b in zip((out, S, A), eager)]
    _say(f"[parity] two stream groups d={d}: out, S_T, A_T bitwise equal to one launch: {same}")
    assert all(same)
