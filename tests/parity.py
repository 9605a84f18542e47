"""Shared helpers of the parity tests: relative L2 and the oracle over chosen streams."""

import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

from oracle import vla_forward as oracle_forward
from rls_associative_memory_amd.inputs import make_stream

TOL = {"f32": 1e-4, "bf16": 1e-2}


def rel_l2(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def _one(args):
    w, s = args
    q, k, v, u = make_stream(w, s)
    return oracle_forward(q, k, v, u, w.lambda0, eps=w.eps)


def oracle_streams(w, streams, workers=None):
    """Oracle (out, S_T, A_T) for each listed stream, computed in worker processes."""
    streams = list(streams)
    if workers is None:
        workers = min(len(streams), max(1, min(16, os.cpu_count() or 1)))
    if workers <= 1 or len(streams) == 1:
        return [_one((w, s)) for s in streams]
    with ProcessPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(_one, [(w, s) for s in streams]))
