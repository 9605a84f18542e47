"""C-ABI library: loads, exports what include/vla.h declares, rejects bad arguments.

The CPU cases never launch work: every call here fails argument validation, which the
library performs before it touches a device.
"""

import ctypes

import pytest
import torch

from rls_associative_memory_amd import vla


@pytest.fixture(scope="module")
def lib():
    return vla.load_library()


def desc(**kw):
    base = dict(B=2, H=3, T=17, d=64, dtype=1, path=0, eps=1e-6, chunk=0, workspace=None,
                workspace_bytes=0, gain=0)
    base.update(kw)
    return vla.VlaDesc(**base)


def test_header_symbols_are_exported(lib):
    names = vla.exported_symbols()
    assert {"vla_forward", "vla_workspace_size", "vla_status_string", "vla_resolve_path",
            "vla_version"} <= set(names)
    for name in names:
        assert hasattr(lib, name), f"{name} declared in include/vla.h but not exported"


def test_status_strings_and_version(lib):
    for code, name in vla.STATUS.items():
        assert lib.vla_status_string(code).decode() == name
    assert lib.vla_status_string(99).decode() == "VLA_ERROR_UNKNOWN"
    assert lib.vla_version() >= 100


@pytest.mark.parametrize("bad", [
    dict(B=0), dict(H=-1), dict(T=0), dict(d=0), dict(dtype=7), dict(path=9), dict(eps=-1.0),
    dict(eps=float("nan")), dict(eps=float("inf")), dict(chunk=-4), dict(B=1 << 40, H=1 << 40),
])
def test_invalid_descriptors(lib, bad):
    n = ctypes.c_size_t(123)
    assert lib.vla_workspace_size(ctypes.byref(desc(**bad)), ctypes.byref(n)) == 1
    p = ctypes.c_int32(0)
    assert lib.vla_resolve_path(ctypes.byref(desc(**bad)), ctypes.byref(p)) == 1


@pytest.mark.parametrize("d", [1, 16, 48, 80, 256])
def test_unsupported_head_dim(lib, d):
    n = ctypes.c_size_t(0)
    assert lib.vla_workspace_size(ctypes.byref(desc(d=d)), ctypes.byref(n)) == 2


def test_null_out_params(lib):
    assert lib.vla_workspace_size(ctypes.byref(desc()), None) == 1
    assert lib.vla_resolve_path(ctypes.byref(desc()), None) == 1
    assert lib.vla_workspace_size(None, ctypes.byref(ctypes.c_size_t(0))) == 1


def test_forward_argument_errors_before_any_device_work(lib):
    ok = desc()
    nul = None
    fake = 4096  # never dereferenced: every call below fails validation first
    # NULL required pointers
    for i in range(5):
        ptrs = [fake] * 5
        ptrs[i] = nul
        q, k, v, u, out = ptrs
        assert lib.vla_forward(q, k, v, u, 1.0, out, None, None, ctypes.byref(ok), None) == 1
    # lambda0 <= 0 or not finite
    for lam in (0.0, -1.0, float("nan"), float("inf")):
        assert lib.vla_forward(fake, fake, fake, fake, lam, fake, None, None,
                               ctypes.byref(ok), None) == 1
    # NULL descriptor
    assert lib.vla_forward(fake, fake, fake, fake, 1.0, fake, None, None, None, None) == 1
    # misaligned pointers
    assert lib.vla_forward(fake + 2, fake, fake, fake, 1.0, fake, None, None,
                           ctypes.byref(ok), None) == 2
    assert lib.vla_forward(fake, fake, fake, fake, 1.0, fake, None, fake + 8,
                           ctypes.byref(ok), None) == 2


def test_forward_state_argument_errors_before_any_device_work(lib):
    ok = desc()
    fake = 4096  # never dereferenced
    call = lambda lam, S0=None, A0=None, n0=None, nf=None, q=fake: lib.vla_forward_state(
        q, fake, fake, fake, lam, S0, A0, n0, fake, None, None, nf, ctypes.byref(ok), None)
    assert call(1.0, q=None) == 1                       # NULL input
    for lam in (0.0, float("nan")):
        assert call(lam) == 1                           # lambda0 checked when A0 is NULL
    for kw in ({"S0": fake + 4}, {"A0": fake + 8}, {"n0": fake + 2}, {"nf": fake + 12}):
        assert call(1.0, **kw) == 2                     # misaligned state pointers


def test_forward_state_binding_checks_state_tensors():
    x = torch.zeros(1, 1, 4, 32)
    with pytest.raises(ValueError):
        vla.forward_state(x, x, x, x, 1.0)
    if torch.cuda.is_available():  # shapes are checked before the library is called
        y = x.cuda()
        with pytest.raises(ValueError):
            vla.forward_state(y, y, y, y, 1.0, n0=torch.zeros(1, 1, 31, device="cuda"))


def test_forward_state_rejects_in_place_state(lib):
    """Output state overlapping input state is an argument error (checked on the host).

    The pointers are fake: without the check the call would return VLA_ERROR_NO_DEVICE on a
    machine without a GPU, and on one with a GPU it would launch, so it runs without one only.
    """
    if torch.cuda.is_available():
        pytest.skip("fake device pointers are only passed where no GPU can be reached")
    d = desc(B=1, H=2, T=8, d=32)
    mat = 2 * 32 * 32 * 4
    base = 1 << 20
    fake = lambda off: ctypes.c_void_p(base + off)
    args = [fake(0)] * 4
    # A_final == A0
    assert lib.vla_forward_state(*args, ctypes.c_float(1.0), fake(mat), fake(2 * mat), None,
                                 fake(8 * mat), None, fake(2 * mat), None, ctypes.byref(d), None) == 1
    # n_final inside S0
    assert lib.vla_forward_state(*args, ctypes.c_float(1.0), fake(mat), None, None,
                                 fake(8 * mat), None, None, fake(mat + 256), ctypes.byref(d), None) == 1


def test_linear_attention_argument_errors(lib):
    """Argument errors of vla_linear_attention come back before any device work."""
    x = ctypes.c_void_p(1 << 20)
    d = desc(B=1, H=2, T=100, d=64)
    assert lib.vla_linear_attention(None, x, x, x, None, None, ctypes.byref(d), None) == 1
    assert lib.vla_linear_attention(x, x, x, x, None, None, ctypes.byref(desc(d=48)), None) == 2
    assert lib.vla_linear_attention(x, x, x, x, None, None, ctypes.byref(desc(path=1)), None) == 2
    assert lib.vla_linear_attention(x, x, x, x, None, None, ctypes.byref(desc(chunk=32)), None) == 2
    assert lib.vla_linear_attention(ctypes.c_void_p((1 << 20) + 8), x, x, x, None, None,
                                    ctypes.byref(d), None) == 2
    small = desc(B=1, H=2, T=100, d=64, workspace=1 << 20, workspace_bytes=16)
    assert lib.vla_linear_attention(x, x, x, x, None, None, ctypes.byref(small), None) == 1
    n = ctypes.c_size_t(0)
    assert lib.vla_la_workspace_size(ctypes.byref(d), ctypes.byref(n)) == 0
    # 2 streams x 2 segments (one chunk each) x (d^2 + d) fp32
    assert n.value == 2 * 2 * (64 * 64 + 64) * 4
    assert lib.vla_la_workspace_size(ctypes.byref(desc(path=2)), ctypes.byref(n)) == 2


def test_raw_gain_descriptor(lib):
    p = ctypes.c_int32(-1)
    assert lib.vla_resolve_path(ctypes.byref(desc(gain=2)), ctypes.byref(p)) == 1
    assert lib.vla_resolve_path(ctypes.byref(desc(gain=-1)), ctypes.byref(p)) == 1
    long = desc(B=1, H=2, T=4096, d=96, gain=1)
    assert lib.vla_resolve_path(ctypes.byref(long), ctypes.byref(p)) == 0
    assert p.value == vla.PATHS["seq"]                    # the chunked path has no raw gain
    assert lib.vla_resolve_path(ctypes.byref(desc(B=1, H=2, T=4096, d=96)), ctypes.byref(p)) == 0
    assert p.value == vla.PATHS["chunk"]
    assert lib.vla_resolve_path(ctypes.byref(desc(T=4096, path=2, gain=1)), ctypes.byref(p)) == 2
    assert lib.vla_resolve_path(ctypes.byref(desc(T=1, gain=1)), ctypes.byref(p)) == 0
    assert p.value == vla.PATHS["decode"]
    n = ctypes.c_size_t(0)
    assert lib.vla_la_workspace_size(ctypes.byref(desc(gain=1)), ctypes.byref(n)) == 2
    with pytest.raises(ValueError):
        vla.make_desc((1, 1, 4, 32), torch.float32, gain="half")


def test_backward_argument_errors(lib):
    """Argument errors of vla_backward come back before any device work."""
    x = ctypes.c_void_p(1 << 20)
    d = desc(B=1, H=2, T=100, d=64)
    f = ctypes.c_float(1.0)
    args = [x, x, x, x, f, x, None, None, None, x, x, x, x, None]
    call = lambda a, dd: lib.vla_backward(*a, ctypes.byref(dd), None)
    bad = list(args); bad[5] = None
    assert call(bad, d) == 1                                   # no d_out
    bad = list(args); bad[4] = ctypes.c_float(0.0)
    assert call(bad, d) == 1                                   # lambda0 <= 0
    assert call(args, desc(B=1, H=2, T=100, d=64, path=3)) == 2    # decode
    assert call(args, desc(B=1, H=2, T=100, d=64, path=2, chunk=48)) == 2
    assert call(args, desc(B=1, H=2, T=100, d=64, gain=1)) == 2
    bad = list(args); bad[9] = ctypes.c_void_p((1 << 20) + 4)
    assert call(bad, d) == 2                                   # misaligned dq
    small = desc(B=1, H=2, T=100, d=64, workspace=1 << 20, workspace_bytes=64)
    assert call(args, small) == 1
    n = ctypes.c_size_t(0)
    assert lib.vla_backward_workspace_size(ctypes.byref(d), ctypes.byref(n)) == 0
    # one segment per stream: T (4 d + 8) floats of records, ceil(T / 64) checkpoints of
    # 2 d^2 floats, ceil(T / 32) S cotangents of d^2 floats, n after the segment, two d x d
    # matrices and one double, per stream, each buffer 256-byte aligned
    al = lambda x: (x + 255) // 256 * 256
    seq = (al(2 * 100 * (4 * 64 + 8) * 4) + al(2 * 2 * 2 * 64 * 64 * 4) + al(2 * 4 * 64 * 64 * 4)
           + al(2 * 64 * 4) + 2 * al(2 * 64 * 64 * 4) + al(2 * 8))
    assert n.value == seq
    assert lib.vla_backward_workspace_size(ctypes.byref(desc(B=1, H=2, T=100, d=64, path=1)),
                                           ctypes.byref(n)) == 0 and n.value == seq
    # few long streams: AUTO splits time (the chunked path's segments, its workspace on top)
    ws = lambda **kw: (lib.vla_backward_workspace_size(ctypes.byref(desc(**kw)), ctypes.byref(n)), n.value)[1]
    long_auto = ws(B=1, H=2, T=4096, d=96)
    assert long_auto == ws(B=1, H=2, T=4096, d=96, path=2) > ws(B=1, H=2, T=4096, d=96, path=1)
    assert ws(B=1, H=1024, T=4096, d=96) == ws(B=1, H=1024, T=4096, d=96, path=2)
    # at d = 128 only up to 128 streams; a split into one segment per stream is SEQ
    assert ws(B=1, H=128, T=2048, d=128) == ws(B=1, H=128, T=2048, d=128, path=2)
    assert ws(B=1, H=129, T=2048, d=128) == ws(B=1, H=129, T=2048, d=128, path=1)
    assert ws(B=1, H=2048, T=512, d=32, dtype=0) == ws(B=1, H=2048, T=512, d=32, dtype=0, path=1)
    assert ws(B=1, H=1024, T=512, d=32, dtype=0) == ws(B=1, H=1024, T=512, d=32, dtype=0, path=2)
    # 256 fp32 streams of 512 tokens (the recall workload): 64-token segments, eight per stream
    assert ws(B=64, H=4, T=512, d=32, dtype=0) == ws(B=64, H=4, T=512, d=32, dtype=0, path=2)


def test_decode_path_resolution(lib):
    p = ctypes.c_int32(-1)
    assert lib.vla_resolve_path(ctypes.byref(desc(T=1)), ctypes.byref(p)) == 0
    assert p.value == vla.PATHS["decode"]                 # AUTO picks decode for T = 1
    assert lib.vla_resolve_path(ctypes.byref(desc(T=1, path=1)), ctypes.byref(p)) == 0
    assert p.value == vla.PATHS["seq"]                    # a forced path is kept
    assert lib.vla_resolve_path(ctypes.byref(desc(T=2, path=3)), ctypes.byref(p)) == 2
    assert lib.vla_resolve_path(ctypes.byref(desc(path=4)), ctypes.byref(p)) == 1
    n = ctypes.c_size_t(99)
    assert lib.vla_workspace_size(ctypes.byref(desc(T=1)), ctypes.byref(n)) == 0 and n.value == 0


def test_sequential_path_needs_no_workspace(lib):
    n = ctypes.c_size_t(99)
    assert lib.vla_workspace_size(ctypes.byref(desc(path=1)), ctypes.byref(n)) == 0
    assert n.value == 0


def test_binding_rejects_host_tensors():
    x = torch.zeros(1, 1, 4, 32)
    with pytest.raises(ValueError):
        vla.forward(x, x, x, x, 1.0)


@pytest.mark.parametrize("shape,dtype,want", [
    ((1, 1, 256, 32), 0, "chunk"),        # one fp32 stream of 256 tokens: 64-token segments
    ((64, 4, 512, 32), 0, "chunk"),       # 256 fp32 streams of 512 tokens (the recall workload)
    ((8, 8, 4096, 64), 1, "chunk"),       # few streams, long sequences
    ((2, 16, 43008, 128), 1, "chunk"),
    ((1, 32, 131072, 96), 1, "chunk"),
    ((64, 8, 512, 32), 0, "seq"),         # 512 fp32 streams fill the machine token by token
    ((64, 4, 512, 32), 1, "seq"),         # bf16 segments are at least 256 tokens
    ((64, 4, 128, 32), 0, "seq"),         # too short to split
    ((8, 4, 1, 96), 1, "decode"),
])
def test_auto_path_choice(lib, shape, dtype, want):
    B, H, T, d = shape
    p = ctypes.c_int32(-1)
    assert lib.vla_resolve_path(ctypes.byref(desc(B=B, H=H, T=T, d=d, dtype=dtype)), ctypes.byref(p)) == 0
    assert p.value == vla.PATHS[want], (shape, dtype, p.value)


def _fake(off):
    return ctypes.c_void_p((1 << 24) + off)


def test_outputs_must_not_alias_inputs(lib):
    """out (or a state output, or a caller's workspace) overlapping an input or another output
    is an argument error, reported before any device work (fake pointers, never touched)."""
    if torch.cuda.is_available():
        pytest.skip("fake device pointers are only passed where no GPU can be reached")
    d = desc(B=1, H=2, T=64, d=32, dtype=0, path=1)
    tok = 2 * 64 * 32 * 4
    mat = 2 * 32 * 32 * 4
    q, k, v, u = (_fake(i * tok) for i in range(4))
    f = ctypes.c_float(1.0)
    fwd = lambda out, S=None, A=None, dd=d: lib.vla_forward(q, k, v, u, f, out, S, A, ctypes.byref(dd), None)
    assert fwd(_fake(2 * tok)) == 1                              # out is v
    assert fwd(_fake(3 * tok + tok // 2)) == 1                   # out starts inside u
    assert fwd(_fake(3 * tok - 256)) == 1                        # out ends inside u
    base = 8 * tok
    assert fwd(_fake(base), S=_fake(base + tok - 16)) == 1       # S_final inside out
    assert fwd(_fake(base), S=_fake(base + tok), A=_fake(base + tok)) == 1   # S_final is A_final
    assert fwd(_fake(base), S=_fake(0)) == 1                     # S_final is q
    # disjoint buffers pass the check and stop only at the device check
    assert fwd(_fake(base), S=_fake(base + tok), A=_fake(base + tok + mat)) == 5
    # a caller's workspace overlapping an output
    ch = desc(B=1, H=2, T=2048, d=32, dtype=0, path=2)
    n = ctypes.c_size_t(0)
    assert lib.vla_workspace_size(ctypes.byref(ch), ctypes.byref(n)) == 0
    tk = 2 * 2048 * 32 * 4
    q2, k2, v2, u2 = (_fake(i * tk) for i in range(4))
    o2 = _fake(4 * tk)
    ws_bad = desc(B=1, H=2, T=2048, d=32, dtype=0, path=2, workspace=(1 << 24) + 4 * tk + 4096,
                  workspace_bytes=n.value)
    assert lib.vla_forward(q2, k2, v2, u2, f, o2, None, None, ctypes.byref(ws_bad), None) == 1
    ws_ok = desc(B=1, H=2, T=2048, d=32, dtype=0, path=2, workspace=(1 << 24) + 5 * tk,
                 workspace_bytes=n.value)
    assert lib.vla_forward(q2, k2, v2, u2, f, o2, None, None, ctypes.byref(ws_ok), None) == 5
    # linear attention: out is k
    la = desc(B=1, H=2, T=64, d=32, dtype=0)
    assert lib.vla_linear_attention(q, k, v, _fake(tok), None, None, ctypes.byref(la), None) == 1
    # backward: a gradient overlapping d_out, and two gradients sharing memory
    dout = _fake(4 * tok)
    g = [_fake(8 * tok + i * tok) for i in range(4)]
    bw = lambda grads: lib.vla_backward(q, k, v, u, f, dout, None, None, None, *grads, None,
                                        ctypes.byref(la), None)
    assert bw([dout, g[1], g[2], g[3]]) == 1
    assert bw([g[0], g[0], g[2], g[3]]) == 1
    assert bw(g) == 5


def test_noalloc_argument_errors(lib):
    """vla_forward_state_noalloc refuses a caller's workspace and a scratch need beyond its
    static array before any device work (fake pointers, never touched)."""
    x = ctypes.c_void_p(1 << 24)
    f = ctypes.c_float(1.0)
    call = lambda dd: lib.vla_forward_state_noalloc(x, x, x, x, f, None, None, None,
                                                     ctypes.c_void_p((1 << 30)), None, None, None,
                                                     ctypes.byref(dd), None)
    assert call(desc(B=1, H=2, T=2048, d=32, dtype=0, path=2, workspace=1 << 28,
                     workspace_bytes=1 << 26)) == 1
    big = desc(B=8, H=8, T=4096, d=64, dtype=1, path=2)
    n = ctypes.c_size_t(0)
    assert lib.vla_workspace_size(ctypes.byref(big), ctypes.byref(n)) == 0
    assert n.value > vla.NOALLOC_SCRATCH_BYTES
    assert call(big) == 2
