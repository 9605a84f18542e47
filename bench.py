"""Throughput of the VLA forward recurrence on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--path auto|seq|chunk]

One step is one ``vla_forward`` call over the whole workload (every (batch, head) stream,
all T tokens, final S and A written when the workload asks for them), with inputs already
resident in HBM.  The timed region is K steps between device synchronisations; the line
printed on stdout is a single JSON object:

  value        tokens*heads per second = B*H*T / seconds per step
  roofline     the whole call's algorithmic FLOP rate (12 d^2 + 20 d flops per token*head,
               the plain count of the recurrence) over the published MI355X FP32 peak, the
               whole call's HBM traffic from the committed rocprofv3 counters beside its
               algorithmic bytes, and the dominant kernel's own rate (its flops per
               token*head over its mean launch time, HIP events on the launch stream)
  precision    how the path's arithmetic is carried out (fp32 state; on bf16 inputs the
               matrix-core operands are two-term bf16 splits)
  cpu_baseline the fp64 oracle timed on the host's cores on a bounded sample of the same
               workload (the first ``--cpu-tokens`` tokens of ``cores`` streams, one process
               per CPU of the affinity mask), whose outputs also give a causal parity check
               of the GPU run's first tokens

Workloads are seeded synthetic inputs (rls_associative_memory_amd.inputs).

``--mode decode`` measures the streaming use instead: every stream of the workload advances
one token per call (T = 1, state carried from call to call through vla_forward_state), and
the line reports token*heads per second of such calls with the HBM rate of the state they
read and write (S and A in, S and A out, per stream per call).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "VLA forward tokens·heads/sec at 1 MI355X; % of FP32/MFMA/HBM roofline"
PEAK_FP32_TFLOPS = 157.3     # MI355X FP32 vector (packed) and FP32 MFMA, dense
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E


def flops_per_token_head(d: int) -> int:
    # z = A u (2d^2), A downdate (2d^2), A khat (2d^2), S khat (2d^2), S update (2d^2),
    # S phi(q) (2d^2), plus the O(d) vector work: 12 d^2 + 20 d.
    return 12 * d * d + 20 * d


# Algorithmic flops per token*head of the work each kernel exists to do, and the unit it
# runs on.  The A side (Sherman-Morrison, gate) and the S side (residual update, readout)
# are each half of the recurrence; the segment map of the chunked path recomputes the
# affine map of the S recurrence over 2d state rows (dot + update per row per token).
KERNEL_WORK = {
    "vla_seq_kernel": (lambda d: 12 * d * d + 20 * d, "alu"),
    "k_aside": (lambda d: 6 * d * d + 10 * d, "alu"),
    "k_aside_wy": (lambda d: 6 * d * d + 10 * d, "mfma"),
    "k_swy_final": (lambda d: 6 * d * d + 10 * d, "mfma"),
    "k_swy_map": (lambda d: 8 * d * d, "mfma"),
    "k_gram": (lambda d: 2 * d * d, "mfma"),
    # linear attention: S update and readout (2 d^2 each) plus the normaliser and ratio
    "k_la_out": (lambda d: 4 * d * d + 6 * d, "mfma"),
    "k_la_seg": (lambda d: 2 * d * d, "mfma"),
}


def bytes_per_token_head(d: int, elem: int) -> int:
    return 5 * d * elem  # q, k, v, u read; out written


PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = os.path.join(ROOT, "rls_associative_memory_amd", "csrc")


# The sources the forward path's kernels and their launches are built from; a change
# anywhere else in csrc/ (the backward, decode or linear-attention kernels) leaves the
# stored counter readings of the forward kernels valid.
FORWARD_SOURCES = ("vla_api.cpp", "vla_chunk.hip", "vla_seq.hip", "vla_aside_wy.h",
                   "vla_swy_bf16.h", "vla_mfma.h", "vla_common.h", "vla_internal.h")


def _code_only(text: str) -> str:
    """C++ source without comments and blank space, so that an edit of comments alone keeps
    the digest (string literals in these sources hold no comment markers)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(root: str = KERNEL_SOURCES) -> str:
    """Digest of the code (comments excluded) of the forward path's HIP sources; a stored
    counter reading is used only while it matches."""
    import hashlib
    h = hashlib.sha256()
    for name in FORWARD_SOURCES:
        with open(os.path.join(root, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary of this workload (profiles/traffic_<workload>.md, lines starting "traffic:"),
    scaled by the copy-kernel calibration stored with it; None if absent or stale."""
    path = os.path.join(PROFILES, f"traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    src = kernel_source_hash()
    with open(path) as f:
        for line in f:
            if not line.startswith("traffic:"):
                continue
            rec = json.loads(line[len("traffic:"):])
            if rec.get("kernel") == kernel and rec.get("source_hash") == src:
                return (rec["fetch_kib"] * rec["fetch_factor"] + rec["write_kib"] * rec["write_factor"]) * 1024
    return None


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=None,
                    help="workload name (default long_t131072_d96; mqar_t512_d32 for --mode backward)")
    ap.add_argument("--path", default="auto", choices=["auto", "seq", "chunk"])
    ap.add_argument("--chunk", type=int, default=-1, help="chunk length (-1: the workload's)")
    ap.add_argument("--cpu-tokens", type=int, default=32768,
                    help="tokens per stream in the oracle sample (0 disables the CPU leg)")
    ap.add_argument("--cpu-cores", type=int, default=0,
                    help="oracle processes (0: every CPU this process may run on, capped by the "
                         "host's per-GPU CPU share in OMP_NUM_THREADS when that is set)")
    ap.add_argument("--mode", default="forward",
                    choices=["forward", "decode", "compare", "ablation", "backward"],
                    help="forward: whole sequences (default); decode: T = 1 calls, state carried; "
                         "compare: VLA, VLA with u = 0 and linear attention on the same inputs; "
                         "ablation: growth of the state-transition product, unit vs raw gain; "
                         "backward: gradients of every input (default workload mqar_t512_d32)")
    ap.add_argument("--bw-seq-steps", type=int, default=1,
                    help="--mode backward on time segments: calls of the one-segment-per-stream path "
                         "timed beside it (0: none)")
    ap.add_argument("--decode-path", default="decode", choices=["decode", "seq"],
                    help="path of the T = 1 calls in --mode decode")
    ap.add_argument("--graph", action="store_true",
                    help="forward mode: capture one call in a HIP graph and time graph replays")
    ap.add_argument("--decode-graph", type=int, default=0,
                    help="decode mode: capture this many (even) T = 1 calls in one HIP graph and "
                         "time graph replays instead of eager calls (0: eager)")
    ap.add_argument("--decode-batch", type=int, default=0,
                    help="batch B of the decode streams (0: the workload's); B x H streams")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="run one device copy of this size first (counter calibration)")
    return ap.parse_args()


def _oracle_job(args):
    os.environ["OMP_NUM_THREADS"] = "1"
    name, stream, T = args
    from oracle import vla_forward as oracle_forward
    from rls_associative_memory_amd.inputs import get_workload, make_stream
    w = get_workload(name)
    q, k, v, u = (x[:T] for x in make_stream(w, stream))
    t0 = time.perf_counter()
    out, _, _ = oracle_forward(q, k, v, u, w.lambda0, eps=w.eps)
    return stream, time.perf_counter() - t0, out


def host_cpus():
    """(processes to use, CPUs this process may run on, os.cpu_count()).  The pool takes every
    CPU of the affinity mask, capped by the per-GPU CPU share that OMP_NUM_THREADS names on a
    shared GPU host."""
    nproc = os.cpu_count() or 1
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = nproc
    share = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    use = min(affinity, share) if share > 0 else affinity
    return max(1, use), affinity, nproc


def cpu_baseline(w, tokens: int, cores: int):
    """The oracle on the first ``tokens`` tokens of ``cores`` streams, one process per
    stream (single-threaded BLAS in each).  Returns the report and the outputs."""
    import multiprocessing as mp
    use, affinity, nproc = host_cpus()
    if cores <= 0:
        cores = use
    tokens = min(tokens, w.T)
    streams = list(range(min(cores, w.streams)))
    env_before = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in env_before:
        os.environ[k] = "1"
    try:
        ctx = mp.get_context("spawn")
        t0 = time.perf_counter()
        with ctx.Pool(processes=len(streams)) as pool:
            res = pool.map(_oracle_job, [(w.name, s, tokens) for s in streams])
        wall = time.perf_counter() - t0
    finally:
        for k, v in env_before.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    work = sum(r[1] for r in res)
    value = len(streams) * tokens / max(max(r[1] for r in res), 1e-9)
    rep = {
        "value": value,
        "unit": "tokens*heads/s",
        "cores": len(streams),
        "nproc": nproc,
        "affinity_cpus": affinity,
        "kind": "oracle",
        "sample": (f"{w.name}: first {tokens} tokens of streams 0..{len(streams) - 1}, one "
                   f"single-threaded fp64 numpy process per stream on {len(streams)} of the "
                   f"host's {nproc} CPUs ({affinity} in this process's affinity mask); "
                   f"{work:.1f} s of CPU work, {wall:.1f} s wall including process start-up"),
    }
    return rep, {r[0]: r[2] for r in res}, tokens


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the VLA streams are independent, so the "
              "multi-GPU split needs no communication and is not run here (use --gpus 1).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from rls_associative_memory_amd import vla
    from rls_associative_memory_amd.inputs import get_workload, upload_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.workload is None:
        args.workload = "mqar_t512_d32" if args.mode == "backward" else "long_t131072_d96"
    w = get_workload(args.workload)
    if args.mode == "backward":
        return backward_bench(args, w)
    if args.mode == "decode":
        return decode_bench(args, w)
    if args.mode == "compare":
        return compare_bench(args, w)
    if args.mode == "ablation":
        return ablation_bench(args)
    chunk = w.chunk if args.chunk < 0 else args.chunk
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calib_copy_mb > 0:
        n = args.calib_copy_mb * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    t_gen = time.perf_counter()
    q, k, v, u = upload_inputs(w, dev)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen
    shape = tuple(q.shape)
    path = vla.resolve_path(shape, q.dtype, path=args.path, chunk=chunk)
    ws_bytes = vla.workspace_size(shape, q.dtype, path=args.path, chunk=chunk)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev) if ws_bytes else None
    out = torch.empty_like(q)
    S = torch.empty((w.B, w.H, w.d, w.d), dtype=torch.float32, device=dev) if w.want_state else None
    A = torch.empty_like(S) if S is not None else None

    def step():
        vla.forward(q, k, v, u, w.lambda0, eps=w.eps, path=args.path, chunk=chunk, out=out,
                    S_final=S, A_final=A, workspace=ws)

    print(f"[bench] workload={w.name} path={path} inputs generated in {t_gen:.1f}s; "
          f"warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    eager_step = step
    if args.graph:
        # one whole call (every kernel of the path) captured once and replayed as a HIP graph;
        # the library's per-kernel events are off inside the graph, so the kernel table below
        # comes from one eager call after the timed replays
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        step = graph.replay

    stream = torch.cuda.current_stream(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    vla.profile_reset()
    vla.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    vla.profile_enable(False)
    kernels = vla.profile_read()
    calls = args.steps  # library calls the kernel table covers
    ev_ms = ev0.elapsed_time(ev1) / args.steps
    ms = max(wall * 1e3 / args.steps, ev_ms)
    if args.graph:  # per-kernel durations from eager calls (events do not run inside the graph)
        vla.profile_reset()
        vla.profile_enable(True)
        calls = 3
        for _ in range(calls):
            eager_step()
        torch.cuda.synchronize()
        vla.profile_enable(False)
        kernels = vla.profile_read()
    tokens = w.B * w.H * w.T
    value = tokens / (ms * 1e-3)
    print(f"[bench] {args.steps} steps: {ms:.3f} ms/step (events {ev_ms:.3f} ms)",
          file=sys.stderr, flush=True)

    for name, (tot, n) in sorted(kernels.items(), key=lambda kv: -kv[1][0]):
        print(f"[bench] kernel {name:16s} {tot / max(n, 1):9.3f} ms/launch x {n}",
              file=sys.stderr, flush=True)
    dom = max(kernels.items(), key=lambda kv: kv[1][0])
    dom_name, (dom_total, dom_n) = dom
    kernel_ms = dom_total / max(dom_n, 1)
    # A large call runs its streams as two groups on two HIP streams: each kernel is then
    # launched once per group, and one launch covers that group's share of the tokens.
    launches_per_call = {name: n / calls for name, (_, n) in kernels.items()}
    dom_per_call = launches_per_call[dom_name]
    tokens_per_launch = tokens / dom_per_call
    work_fn, unit = KERNEL_WORK.get(dom_name, (lambda d: 0, "alu"))
    achieved = work_fn(w.d) * tokens_per_launch / (kernel_ms * 1e-3) / 1e12
    path_tflops = flops_per_token_head(w.d) * tokens / (ms * 1e-3) / 1e12
    alg_bytes = bytes_per_token_head(w.d, w.elem_bytes) * tokens
    if w.want_state:
        alg_bytes += 2 * w.B * w.H * w.d * w.d * 4  # S_T and A_T written
    call_traffic = None
    if path == "chunk":
        per = [stored_traffic(w.name, name) for name in kernels]
        if per and all(x is not None for x in per):
            call_traffic = sum(x * launches_per_call[name] for x, name in zip(per, kernels))
    path_bound = "mfma" if path == "chunk" else "alu"
    roofline = {
        # The whole vla_forward call: F(d) = 12 d^2 + 20 d algorithmic flops per token*head
        # over the step time, against the MI355X FP32 peak (the arithmetic is fp32; on the
        # chunked path it runs on the matrix cores as two-term bf16 products).
        "bound": path_bound,
        "achieved": round(path_tflops, 3),
        "peak": PEAK_FP32_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(path_tflops / PEAK_FP32_TFLOPS, 4),
        "traffic": call_traffic,
        "scope": "whole vla_forward call (every kernel of the path), F(d) = 12 d^2 + 20 d flops per token*head",
        "target_frac": 0.5,
        "algorithmic_bytes": alg_bytes,
        "traffic_over_algorithmic": round(call_traffic / alg_bytes, 3) if call_traffic else None,
        "hbm_frac": round(alg_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "dominant_kernel": {
            "name": dom_name,
            "bound": unit,
            "ms": round(kernel_ms, 4),
            "launches_per_call": round(dom_per_call, 3),
            "tokens_per_launch": tokens_per_launch,
            "timing": "HIP events on the launch stream around each launch, mean over the timed steps"
                      + ("; the call's two stream groups run at the same time on two HIP streams, so "
                         "each launch's window is shared with the other group's kernels"
                         if dom_per_call > 1 else ""),
            "flops_per_token_head": work_fn(w.d),
            "achieved": round(achieved, 3),
            "peak": PEAK_FP32_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP32_TFLOPS, 4),
            "traffic": stored_traffic(w.name, dom_name),
        },
    }
    precision = ("fp32 inputs: fp32 arithmetic throughout" if w.dtype == "f32" else
                 "bf16 inputs (exact in bf16); fp32 state and accumulation; every fp32 operand of a "
                 "matrix-core product split into two bf16 terms (hi + lo, about 16 significant "
                 "bits), the lo x lo term dropped; out rounded once to bf16")
    if path == "seq":
        precision = "fp32 state and arithmetic on the vector ALUs; out rounded once to the input dtype"

    cpu = None
    if args.cpu_tokens > 0:
        cpu, ref, ntok = cpu_baseline(w, args.cpu_tokens, args.cpu_cores)
        o = out.view(-1, w.T, w.d)
        worst = 0.0
        for s, r in ref.items():
            g = o[s, :ntok].double().cpu().numpy()
            worst = max(worst, float(np.linalg.norm(g - r) / np.linalg.norm(r)))
        print(f"[bench] causal parity of the first {ntok} tokens on {len(ref)} streams: "
              f"worst rel L2 {worst:.3e}", file=sys.stderr, flush=True)

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens*heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "precision": precision,
        "data": "synthetic",
        "config": {
            "workload": w.name, "B": w.B, "H": w.H, "T": w.T, "d": w.d,
            "input_dtype": w.dtype, "state_dtype": "f32", "lambda0": w.lambda0,
            "path": path, "chunk": chunk if path == "chunk" else 0,
            "final_state": bool(w.want_state),
            "hip_graph": bool(args.graph),
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def decode_bench(args, w):
    """T = 1 calls over every stream of the workload, state carried (ping-pong buffers)."""
    import torch
    from rls_associative_memory_amd import vla
    from rls_associative_memory_amd.inputs import upload_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    # enough tokens for the eager warm-up and timed calls, or for one captured graph of calls
    nsteps = max(args.warmup + args.steps, args.decode_graph)
    if args.decode_batch > 0:
        w = w.resized(name=f"{w.name}_b{args.decode_batch}", B=args.decode_batch)
    tok = upload_inputs(w.resized(name=w.name + "_decode", T=nsteps), dev)  # [B, H, steps, d]
    steps_in = [[x[:, :, t:t + 1].contiguous() for x in tok] for t in range(nsteps)]
    mat = (w.B, w.H, w.d, w.d)
    st = [(torch.zeros(mat, dtype=torch.float32, device=dev),
           torch.empty(mat, dtype=torch.float32, device=dev),
           torch.zeros((w.B, w.H, w.d), dtype=torch.float32, device=dev)) for _ in range(2)]
    eye = torch.eye(w.d, dtype=torch.float32, device=dev) / w.lambda0
    st[0][1].copy_(eye.expand(mat))
    out = torch.empty_like(steps_in[0][0])

    def step(t):
        S0, A0, n0 = st[t & 1]
        S1, A1, n1 = st[(t & 1) ^ 1]
        vla.forward_state(*steps_in[t], w.lambda0, S0=S0, A0=A0, n0=n0, eps=w.eps, path=args.decode_path,
                          out=out, S_final=S1, A_final=A1, n_final=n1)

    for t in range(args.warmup):
        step(t)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ng = args.decode_graph
    if ng > 0:
        # ng calls (ping-pong state, so the state ends where it started) in one HIP graph; each
        # replay advances every stream by ng tokens (the same ng input tokens each replay)
        if ng % 2:
            raise SystemExit("--decode-graph must be even (the state ping-pongs between two buffers)")
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for t in range(ng):
                step(t)
        reps = max(1, -(-args.steps // ng))
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(reps):
            graph.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ncalls = reps * ng
        ev_ms = ev0.elapsed_time(ev1) / ncalls
        ms = max(wall * 1e3 / ncalls, ev_ms)
        kernel_ms = ev_ms  # per call inside the graph, launch gaps included
        kernels = {}
    else:
        vla.profile_reset()
        vla.profile_enable(True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for t in range(args.warmup, nsteps):
            step(t)
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        vla.profile_enable(False)
        kernels = vla.profile_read()
        ncalls = args.steps
        ev_ms = ev0.elapsed_time(ev1) / args.steps
        ms = max(wall * 1e3 / args.steps, ev_ms)
    streams = w.B * w.H
    kname = "vla_decode_kernel" if args.decode_path == "decode" else "vla_seq_kernel"
    if ng <= 0:
        k_total, k_n = kernels.get(kname, (0.0, 1))
        kernel_ms = k_total / max(k_n, 1)
    # per stream and call: S, A read and written (fp32 d x d each), n read and written,
    # q, k, v, u read and o written in the input dtype
    state_bytes = streams * (4 * w.d * w.d * 4 + 2 * w.d * 4 + 5 * w.d * w.elem_bytes)
    gbs = state_bytes / (kernel_ms * 1e-3) / 1e9 if kernel_ms > 0 else 0.0
    print(f"[bench] decode{' (HIP graph of %d calls)' % ng if ng > 0 else ''}: "
          f"{ncalls} calls of T = 1 over {streams} streams: {ms * 1e3:.1f} us/call "
          f"(events {ev_ms * 1e3:.1f} us, kernel {kernel_ms * 1e3:.1f} us)", file=sys.stderr, flush=True)
    line = {
        "metric": "VLA decode (T = 1 calls, state carried) tokens·heads/sec at 1 MI355X",
        "value": streams / (ms * 1e-3),
        "unit": "tokens*heads/s",
        "n_gpus": 1,
        "steps": ncalls,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name + "_decode", "B": w.B, "H": w.H, "T": 1, "d": w.d,
                   "input_dtype": w.dtype, "state_dtype": "f32", "lambda0": w.lambda0,
                   "path": args.decode_path, "hip_graph_calls": ng if ng > 0 else None},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "kernel": kname, "kernel_ms": round(kernel_ms, 5)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def _time_calls(fn, steps, warmup):
    """Milliseconds per call (max of wall clock and stream events) and the per-kernel
    table of the timed calls."""
    import torch
    from rls_associative_memory_amd import vla
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    vla.profile_reset()
    vla.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        fn()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    vla.profile_enable(False)
    kernels = vla.profile_read()
    return max(wall * 1e3 / steps, ev0.elapsed_time(ev1) / steps), kernels


def compare_bench(args, w):
    """VLA, VLA with u = 0 (the delta rule with unit gains) and the linear-attention
    baseline on the same resident inputs: the wall-clock price of the Sherman-Morrison
    update that the pages put at about five times linear attention's operations."""
    import torch
    from rls_associative_memory_amd import vla
    from rls_associative_memory_amd.inputs import upload_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v, u = upload_inputs(w, dev)
    u0 = torch.zeros_like(u)
    out = torch.empty_like(q)
    shape = tuple(q.shape)
    chunk = w.chunk if args.chunk < 0 else args.chunk
    ws_v = vla.workspace_size(shape, q.dtype, path=args.path, chunk=chunk)
    ws_l = vla.la_workspace_size(shape, q.dtype)
    ws = torch.empty(max(ws_v, ws_l, 16), dtype=torch.uint8, device=dev)
    S = torch.empty((w.B, w.H, w.d, w.d), dtype=torch.float32, device=dev)
    A = torch.empty_like(S)
    n = torch.empty((w.B, w.H, w.d), dtype=torch.float32, device=dev)
    tokens = w.B * w.H * w.T
    res = {}
    for name, fn in (
            ("vla", lambda: vla.forward(q, k, v, u, w.lambda0, eps=w.eps, path=args.path, chunk=chunk,
                                        out=out, S_final=S, A_final=A, workspace=ws)),
            ("vla_u0", lambda: vla.forward(q, k, v, u0, w.lambda0, eps=w.eps, path=args.path,
                                           chunk=chunk, out=out, S_final=S, A_final=A, workspace=ws)),
            ("la", lambda: vla.linear_attention(q, k, v, eps=w.eps, out=out, S_final=S, n_final=n,
                                                workspace=ws))):
        ms, kernels = _time_calls(fn, args.steps, args.warmup)
        res[name] = (ms, kernels)
        print(f"[bench] {name}: {ms:.3f} ms/call", file=sys.stderr, flush=True)
        for kn, (tot, cnt) in sorted(kernels.items(), key=lambda kv: -kv[1][0]):
            print(f"[bench]   kernel {kn:16s} {tot / max(cnt, 1):9.3f} ms/launch x {cnt}",
                  file=sys.stderr, flush=True)
    la_ms, la_k = res["la"]
    k_tot, k_n = la_k.get("k_la_out", (0.0, 1))
    kernel_ms = k_tot / max(k_n, 1)
    achieved = KERNEL_WORK["k_la_out"][0](w.d) * tokens / (kernel_ms * 1e-3) / 1e12 if kernel_ms else 0.0
    line = {
        "metric": "linear attention (same harness) tokens·heads/sec at 1 MI355X; VLA / LA time ratio",
        "value": tokens / (la_ms * 1e-3),
        "unit": "tokens*heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": la_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "d": w.d, "input_dtype": w.dtype},
        "compare": {
            "vla_ms": round(res["vla"][0], 4),
            "vla_u0_ms": round(res["vla_u0"][0], 4),
            "la_ms": round(la_ms, 4),
            "vla_over_la_time": round(res["vla"][0] / la_ms, 3),
            "vla_over_la_flops": round(flops_per_token_head(w.d) / (4 * w.d * w.d + 6 * w.d), 3),
        },
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_FP32_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP32_TFLOPS, 4),
                     "traffic": None, "kernel": "k_la_out", "kernel_ms": round(kernel_ms, 4)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def backward_bench(args, w):
    """vla_backward over a whole workload (random cotangents for out, S_T, A_T, n_T): one
    step is one call, on --path (auto: time segments for few long streams, else one segment
    per stream).  When the call runs on time segments, the one-segment-per-stream call is
    timed beside it (--bw-seq-steps calls, after one warm-up).  Work per token*head is counted
    as the kernels execute it, two flops per multiply-add: the forward (token by token, or the
    chunked forward passes) 12 d^2; the S cotangent sweep 6 d^2; the chunked gradient pass
    14 d^2 of products with a d x d operand plus 704 d of products within its 32-token chunks
    (the 32 x 32 matrices: 5 of 2 * 32 d each, and 8 triangular products of about 3/4 of
    2 * 32 d each); on time segments the du correction 2 d^2 (the segment maps' 6 d^2 are left
    out of the count)."""
    import torch
    from rls_associative_memory_amd import vla
    from rls_associative_memory_amd.inputs import upload_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v, u = upload_inputs(w, dev)
    g = torch.Generator(device=dev).manual_seed(3)
    d_out = torch.randn(q.shape, generator=g, device=dev).to(q.dtype)
    mat = (w.B, w.H, w.d, w.d)
    dS = torch.randn(mat, generator=g, device=dev)
    dA = torch.randn(mat, generator=g, device=dev)
    dn = torch.randn((w.B, w.H, w.d), generator=g, device=dev)
    shape = tuple(q.shape)
    tokens = w.B * w.H * w.T

    def run(path, steps, warmup):
        ws = torch.empty(vla.backward_workspace_size(shape, q.dtype, path=path), dtype=torch.uint8, device=dev)
        ms, kernels = _time_calls(lambda: vla.backward(q, k, v, u, w.lambda0, d_out, dS, dA, dn, eps=w.eps,
                                                       workspace=ws, path=path), steps, warmup)
        del ws
        torch.cuda.empty_cache()
        return ms, kernels

    ms, kernels = run(args.path, args.steps, args.warmup)
    segmented = "k_bw_dsmap" in kernels or "k_bw_fix" in kernels
    print(f"[bench] backward {w.name} ({'time segments' if segmented else 'one segment per stream'}): "
          f"{ms:.3f} ms/call", file=sys.stderr, flush=True)
    for kn, (tot, cnt) in sorted(kernels.items(), key=lambda kv: -kv[1][0]):
        print(f"[bench]   kernel {kn:16s} {tot / max(cnt, 1):9.3f} ms/launch x {cnt}", file=sys.stderr, flush=True)
    d2 = w.d * w.d
    flops = ((12 + 6 + 14) * d2 + 704 * w.d) * tokens
    if segmented:
        flops += 2 * d2 * tokens  # the segment maps' 6 d^2 (not on the first segment) are not counted
    achieved = flops / (ms * 1e-3) / 1e12
    seq = None
    if segmented and args.bw_seq_steps > 0:
        seq_ms, seq_k = run("seq", args.bw_seq_steps, 1)
        print(f"[bench] backward {w.name} (one segment per stream): {seq_ms:.3f} ms/call", file=sys.stderr,
              flush=True)
        seq = {"ms_per_call": round(seq_ms, 3), "calls": args.bw_seq_steps,
               "tokens_heads_per_s": tokens / (seq_ms * 1e-3),
               "kernels_ms": {kn: round(tot / max(cnt, 1), 3) for kn, (tot, cnt) in seq_k.items()},
               "speedup_of_segments": round(seq_ms / ms, 2)}
    line = {
        "metric": "VLA backward (dq, dk, dv, du, dlambda0) tokens·heads/sec at 1 MI355X",
        "value": tokens / (ms * 1e-3),
        "unit": "tokens*heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "d": w.d, "input_dtype": w.dtype,
                   "path": "segments" if segmented else "seq"},
        "roofline": {"bound": "alu", "achieved": round(achieved, 3), "peak": PEAK_FP32_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP32_TFLOPS, 4), "traffic": None,
                     "scope": "whole vla_backward call, executed flops (see the docstring)"},
        "kernels_ms": {kn: round(tot / max(cnt, 1), 3) for kn, (tot, cnt) in kernels.items()},
        "sequential": seq,
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


LAMBDAS = (0.001, 0.01, 0.05, 0.25, 1.0, 4.0)


def ablation_bench(args):
    """Norm of the state-transition product prod_t (I - khat_t g_t^T) after 25, 100 and 1000
    tokens, with the unit gain g = ahat (the method) and the raw gain g = A_t khat (the
    ablation of VLA summary §3.1, Prop. 2), over head sizes and lambda0.

    The product is the state itself: the recurrence with v = 0 from S_0 = I (carried state)
    on the sequential kernel, continued from call to call.  Inputs: 64 streams of i.i.d.
    N(0, 1) q, k, u (the recipe of the other workloads), fp32.  Spectral norms in fp64 on
    the host.  One JSON line: the median and maximum over the streams per configuration."""
    import torch
    from rls_associative_memory_amd import vla
    from rls_associative_memory_amd.inputs import Workload, upload_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    checkpoints = (25, 100, 1000)
    streams = 64
    rows = []
    t_all = time.perf_counter()
    for d in (32, 64, 96, 128):
        w = Workload(f"ablation_d{d}", 1, streams, checkpoints[-1], d, "f32", 1.0, 7, "iid")
        q, k, v, u = upload_inputs(w, dev)
        v.zero_()
        eye = torch.eye(d, dtype=torch.float32, device=dev).expand(1, streams, d, d).contiguous()
        for lam in LAMBDAS:
            for gain in ("unit", "raw"):
                S, A, n = eye, None, None
                t0 = 0
                rec = {"d": d, "lambda0": lam, "gain": gain}
                for t1 in checkpoints:
                    part = [x[:, :, t0:t1].contiguous() for x in (q, k, v, u)]
                    _, S, A, n = vla.forward_state(*part, lam, S0=S, A0=A, n0=n, gain=gain, path="seq")
                    torch.cuda.synchronize()
                    mats = S.view(streams, d, d).double().cpu().numpy()
                    norms = np.array([np.linalg.norm(m, 2) if np.all(np.isfinite(m)) else np.inf
                                      for m in mats])
                    finite = norms[np.isfinite(norms)]
                    rec[f"t{t1}"] = {"median": float(np.median(norms)), "max": float(np.max(norms)),
                                     "finite_streams": int(finite.size)}
                    t0 = t1
                rows.append(rec)
                print(f"[bench] ablation d={d} lambda0={lam} {gain}: "
                      + " ".join(f"t={c}: {rec[f't{c}']['median']:.3e}" for c in checkpoints),
                      file=sys.stderr, flush=True)
    line = {
        "metric": "||prod_t (I - khat_t g_t^T)||_2 after 25/100/1000 tokens, unit vs raw gain (median over 64 streams)",
        "value": None,
        "unit": "spectral norm",
        "n_gpus": 1,
        "data": "synthetic",
        "dtype": "f32",
        "config": {"workload": "ablation_iid_64streams_t1000", "streams": streams, "d": [32, 64, 96, 128],
                   "lambda0": list(LAMBDAS), "checkpoints": list(checkpoints), "path": "seq"},
        "seconds": round(time.perf_counter() - t_all, 1),
        "table": rows,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
