"""The allocation-free entry point, vla_forward_state_noalloc, against vla_forward_state.

Both run the same kernels; the allocation-free call takes the chunked path's scratch from the
library's static per-GPU array instead of a workspace or the library's cache.  Two calls in a
row (the second on a smaller input, so the array holds the first call's contents when it
starts) must each equal vla_forward_state's result bitwise, the outputs being deterministic.
"""

import sys

import numpy as np
import pytest
import torch

from rls_associative_memory_amd import vla
from rls_associative_memory_amd.inputs import get_workload, upload_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _inputs(name, **kw):
    w = get_workload(name).resized(name=f"noalloc_{name}", **kw)
    return w, upload_inputs(w, "cuda")


def _both(w, dev, path, state=None):
    S0, A0, n0 = state if state is not None else (None, None, None)
    ref = vla.forward_state(*dev, w.lambda0, S0=S0, A0=A0, n0=n0, eps=w.eps, path=path)
    got = vla.forward_state(*dev, w.lambda0, S0=S0, A0=A0, n0=n0, eps=w.eps, path=path, noalloc=True)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_equals_forward_state_two_calls():
    # first call: 4 streams of 6000 bf16 tokens, d = 96, chunked (scratch ~25 MiB)
    w1, dev1 = _inputs("long_t131072_d96", B=1, H=4, T=6000)
    need1 = vla.workspace_size(tuple(dev1[0].shape), dev1[0].dtype, path="chunk")
    assert 0 < need1 <= vla.NOALLOC_SCRATCH_BYTES
    _say(f"[case] noalloc call 1: bf16 1x4x6000x96 chunked, scratch {need1 / 2**20:.1f} MiB")
    ref, got = _both(w1, dev1, "chunk")
    for name, a, b in zip(("out", "S_T", "A_T", "n_T"), ref, got):
        assert torch.equal(a, b), f"call 1: {name} differs from vla_forward_state"
    # second call: fewer, shorter fp32 streams continuing from a carried state
    w2, dev2 = _inputs("mqar_t512_d32", B=1, H=2, T=900, d=64)
    need2 = vla.workspace_size(tuple(dev2[0].shape), dev2[0].dtype, path="chunk")
    assert 0 < need2 < need1
    half = [x[:, :, :300].contiguous() for x in dev2]
    rest = [x[:, :, 300:].contiguous() for x in dev2]
    _, S0, A0, n0 = vla.forward_state(*half, w2.lambda0, eps=w2.eps, path="chunk")
    torch.cuda.synchronize()
    _say(f"[case] noalloc call 2: fp32 1x2x600x64 chunked from a carried state, scratch {need2 / 2**20:.2f} MiB")
    ref, got = _both(w2, rest, "chunk", state=(S0, A0, n0))
    for name, a, b in zip(("out", "S_T", "A_T", "n_T"), ref, got):
        assert torch.equal(a, b), f"call 2: {name} differs from vla_forward_state"
    _say("[parity] noalloc: both calls bitwise equal to vla_forward_state")


def test_noalloc_paths_without_scratch_and_limits():
    w, dev = _inputs("iid_t4096_d64", B=2, H=2, T=64)
    _say("[case] noalloc sequential path, 4 x 64 bf16 tokens")
    ref, got = _both(w, dev, "seq")
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    one = [x[:, :, :1].contiguous() for x in dev]
    _say("[case] noalloc decode path, T = 1")
    ref, got = _both(w, one, "auto")
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    # a shape whose scratch exceeds the array is refused before any device work
    big = (8, 8, 4096, 64)
    assert vla.workspace_size(big, torch.bfloat16, path="chunk") > vla.NOALLOC_SCRATCH_BYTES
    wb = get_workload("iid_t4096_d64")
    x = torch.empty(big, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(vla.VlaError) as exc:
        vla.forward_state(x, x, x, x, wb.lambda0, path="chunk", noalloc=True)
    assert exc.value.status == 2
    with pytest.raises(vla.VlaError) as exc:
        ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
        vla.forward_state(*dev, w.lambda0, path="chunk", workspace=ws, noalloc=True)
    assert exc.value.status == 1
    torch.cuda.synchronize()
