"""Seeded synthetic inputs for the VLA forward recurrence.

This module holds none of the method's arithmetic: it only draws q, k, v, u for each
(batch, head) stream, imposes the workload's structure, and rounds to the input dtype.
Both the HIP path (through the tests and the benchmark) and the fp64 oracle consume
exactly these arrays, so the two always see identically rounded inputs.

Streams are generated independently from ``numpy.random.default_rng([seed, stream])``,
so any single stream of a large workload can be regenerated on its own (the parity
tests at full size check sampled streams this way).  Draw order per stream: q, k, v, u
as float32 N(0, 1) arrays of shape [T, d], then any extra noise; structure is imposed
next and the cast to the input dtype (round to nearest even) comes last.

Workloads (sizes from the method's use cases; the summary gives shapes only for the
associative-recall task, VLA summary §4):
  tiny_t256_d32       1 x 1 x 256 x 32,  fp32, lambda0 1    i.i.d. N(0,1)
  mqar_t512_d32       64 x 4 x 512 x 32, fp32, lambda0 1    associative-recall layout:
                      24 unit key/value pairs written at t = 0..23, queried at 24 sorted
                      random positions in [24, T) in a random order, u_t = k_t, all other
                      entries N(0,1) (shape of the n=24, d_h=32 task of §4; no task data)
  iid_t4096_d64       8 x 8 x 4096 x 64, bf16, lambda0 1    i.i.d. N(0,1)
  crossover_t43008_d128  2 x 16 x 43008 x 128, bf16, lambda0 1, u_t = k_t + 0.1 N(0,1)
                      (T near the ~43k-token latency crossover quoted in §3.3)
  long_t131072_d96    1 x 32 x 131072 x 96, bf16, lambda0 0.5, chunk 64, final S and A
"""

from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get_workload", "round_to_bf16", "make_stream",
           "make_inputs", "bf16_bits"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    d: int
    dtype: str          # "f32" or "bf16"
    lambda0: float
    seed: int
    kind: str           # "iid", "mqar", "noisy_u"
    eps: float = 1e-6
    chunk: int = 0      # 0 = let the library choose
    n_pairs: int = 24
    noise: float = 0.1
    want_state: bool = False

    @property
    def streams(self) -> int:
        return self.B * self.H

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def resized(self, **kw) -> "Workload":
        """The same recipe at another size (used by parity tests on small shapes)."""
        return replace(self, **kw)


WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny_t256_d32", 1, 1, 256, 32, "f32", 1.0, 1, "iid"),
        Workload("mqar_t512_d32", 64, 4, 512, 32, "f32", 1.0, 2, "mqar"),
        Workload("iid_t4096_d64", 8, 8, 4096, 64, "bf16", 1.0, 3, "iid"),
        Workload("crossover_t43008_d128", 2, 16, 43008, 128, "bf16", 1.0, 4, "noisy_u"),
        Workload("long_t131072_d96", 1, 32, 131072, 96, "bf16", 0.5, 5, "iid", chunk=64,
                 want_state=True),
    )
}


def get_workload(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}") from None


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    nan = np.isnan(x)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    rounded = np.where(nan, bits | np.uint32(0x00400000), rounded)
    return rounded.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The uint16 bit patterns of bf16-representable float32 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _unit_rows(x: np.ndarray) -> np.ndarray:
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def make_stream(w: Workload, stream: int):
    """q, k, v, u for one stream as float32 [T, d] arrays, already rounded to ``w.dtype``."""
    if not 0 <= stream < w.streams:
        raise IndexError("stream index out of range")
    rng = np.random.default_rng([w.seed, stream])
    T, d = w.T, w.d
    q = rng.standard_normal((T, d), dtype=np.float32)
    k = rng.standard_normal((T, d), dtype=np.float32)
    v = rng.standard_normal((T, d), dtype=np.float32)
    u = rng.standard_normal((T, d), dtype=np.float32)
    if w.kind == "iid":
        pass
    elif w.kind == "noisy_u":
        eta = rng.standard_normal((T, d), dtype=np.float32)
        if w.dtype == "bf16":
            k = round_to_bf16(k)
        u = (k + np.float32(w.noise) * eta).astype(np.float32)
    elif w.kind == "mqar":
        n = min(w.n_pairs, T // 2)
        keys = _unit_rows(rng.standard_normal((n, d), dtype=np.float32)).astype(np.float32)
        vals = _unit_rows(rng.standard_normal((n, d), dtype=np.float32)).astype(np.float32)
        qpos = np.sort(rng.choice(np.arange(n, T), size=n, replace=False))
        perm = rng.permutation(n)
        k[:n] = keys
        v[:n] = vals
        q[qpos] = keys[perm]
        u = k.copy()
    else:
        raise ValueError(f"unknown workload kind {w.kind!r}")
    if w.dtype == "bf16":
        q, k, v, u = (round_to_bf16(x) for x in (q, k, v, u))
    elif w.dtype != "f32":
        raise ValueError("dtype must be 'f32' or 'bf16'")
    return q, k, v, u


def make_inputs(w: Workload, streams=None):
    """Stacked inputs [S, T, d] (float32 arrays) for the given stream indices (default all)."""
    idx = range(w.streams) if streams is None else list(streams)
    parts = [make_stream(w, s) for s in idx]
    return tuple(np.stack([p[i] for p in parts]) for i in range(4))


def torch_dtype(w: Workload):
    import torch
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def upload_inputs(w: Workload, device="cuda", streams=None):
    """Device tensors q, k, v, u of shape [B, H, T, d] (or [len(streams), 1, T, d] for a
    subset) in the workload's dtype, filled stream by stream to bound host memory."""
    import torch
    idx = list(range(w.streams)) if streams is None else list(streams)
    shape = (w.B, w.H, w.T, w.d) if streams is None else (len(idx), 1, w.T, w.d)
    dt = torch_dtype(w)
    bufs = [torch.empty(shape, dtype=dt, device=device) for _ in range(4)]
    flat = [b.view(-1, w.T, w.d) for b in bufs]
    for slot, s in enumerate(idx):
        for buf, x in zip(flat, make_stream(w, s)):
            buf[slot].copy_(torch.from_numpy(x).to(dt))
    return tuple(bufs)
