"""Thin ctypes binding of ``librls_vla.so`` (argument marshalling only).

Every step of the recurrence runs in the library's HIP kernels; torch is used here only to
hold device memory and to name the current HIP stream.  If the library has not been built
the first call raises: there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os
import re
import threading
from typing import Optional

import torch

__all__ = ["forward", "forward_state", "NOALLOC_SCRATCH_BYTES", "backward", "backward_workspace_size", "linear_attention", "la_workspace_size", "workspace_size", "resolve_path", "library_path", "load_library",
           "profile_enable", "profile_reset", "profile_read",
           "VlaError", "exported_symbols", "STATUS", "PATHS", "DTYPES", "GAINS", "VlaDesc"]

STATUS = {
    0: "VLA_SUCCESS",
    1: "VLA_ERROR_INVALID_VALUE",
    2: "VLA_ERROR_NOT_SUPPORTED",
    3: "VLA_ERROR_OUT_OF_MEMORY",
    4: "VLA_ERROR_LAUNCH",
    5: "VLA_ERROR_NO_DEVICE",
}
PATHS = {"auto": 0, "seq": 1, "chunk": 2, "decode": 3}
DTYPES = {torch.float32: 0, torch.bfloat16: 1}
GAINS = {"unit": 0, "raw": 1}  # raw: A_t khat without the normalisation (ablation only)

NOALLOC_SCRATCH_BYTES = 64 << 20  # VLA_NOALLOC_SCRATCH_BYTES in include/vla.h

_PKG = os.path.dirname(os.path.abspath(__file__))
_HEADER = os.path.join(os.path.dirname(_PKG), "include", "vla.h")


class VlaError(RuntimeError):
    def __init__(self, status: int, where: str = "vla_forward"):
        self.status = status
        super().__init__(f"{where} failed: {STATUS.get(status, status)}")


class VlaDesc(ctypes.Structure):
    """Mirror of ``vla_desc_t`` in include/vla.h."""
    _fields_ = [
        ("B", ctypes.c_int64), ("H", ctypes.c_int64), ("T", ctypes.c_int64), ("d", ctypes.c_int64),
        ("dtype", ctypes.c_int32), ("path", ctypes.c_int32), ("eps", ctypes.c_float),
        ("chunk", ctypes.c_int32), ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t), ("gain", ctypes.c_int32),
    ]


def library_path() -> str:
    return os.environ.get("RLS_VLA_LIB", os.path.join(_PKG, "lib", "librls_vla.so"))


_lib = None
_lib_lock = threading.Lock()


def load_library():
    """Open the library once; raises if it is missing (build it first)."""
    global _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        path = library_path()
        if not os.path.exists(path):
            raise FileNotFoundError(
                f"{path} is missing: build it with `python -m rls_associative_memory_amd.build`")
        lib = ctypes.CDLL(path)
        vp = ctypes.c_void_p
        lib.vla_forward.argtypes = [vp, vp, vp, vp, ctypes.c_float, vp, vp, vp,
                                    ctypes.POINTER(VlaDesc), vp]
        lib.vla_forward.restype = ctypes.c_int
        lib.vla_forward_state.argtypes = [vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, vp, vp, vp,
                                          ctypes.POINTER(VlaDesc), vp]
        lib.vla_forward_state.restype = ctypes.c_int
        lib.vla_forward_state_noalloc.argtypes = lib.vla_forward_state.argtypes
        lib.vla_forward_state_noalloc.restype = ctypes.c_int
        lib.vla_linear_attention.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.POINTER(VlaDesc), vp]
        lib.vla_linear_attention.restype = ctypes.c_int
        lib.vla_backward.argtypes = [vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                     ctypes.POINTER(VlaDesc), vp]
        lib.vla_backward.restype = ctypes.c_int
        lib.vla_backward_workspace_size.argtypes = [ctypes.POINTER(VlaDesc), ctypes.POINTER(ctypes.c_size_t)]
        lib.vla_backward_workspace_size.restype = ctypes.c_int
        lib.vla_la_workspace_size.argtypes = [ctypes.POINTER(VlaDesc), ctypes.POINTER(ctypes.c_size_t)]
        lib.vla_la_workspace_size.restype = ctypes.c_int
        lib.vla_workspace_size.argtypes = [ctypes.POINTER(VlaDesc), ctypes.POINTER(ctypes.c_size_t)]
        lib.vla_workspace_size.restype = ctypes.c_int
        lib.vla_resolve_path.argtypes = [ctypes.POINTER(VlaDesc), ctypes.POINTER(ctypes.c_int32)]
        lib.vla_resolve_path.restype = ctypes.c_int
        lib.vla_status_string.argtypes = [ctypes.c_int]
        lib.vla_status_string.restype = ctypes.c_char_p
        lib.vla_version.argtypes = []
        lib.vla_version.restype = ctypes.c_int32
        lib.vla_profile_enable.argtypes = [ctypes.c_int32]
        lib.vla_profile_enable.restype = ctypes.c_int
        lib.vla_profile_reset.argtypes = []
        lib.vla_profile_reset.restype = ctypes.c_int
        lib.vla_profile_count.argtypes = []
        lib.vla_profile_count.restype = ctypes.c_int32
        lib.vla_profile_get.argtypes = [ctypes.c_int32, ctypes.c_char_p, ctypes.c_size_t,
                                        ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_int64)]
        lib.vla_profile_get.restype = ctypes.c_int
        _lib = lib
        return lib


def exported_symbols():
    """Names of the functions include/vla.h declares."""
    with open(_HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vla_[a-z_0-9]+)\s*\(", text)))


def make_desc(shape, dtype, eps=1e-6, path="auto", chunk=0, workspace=None, gain="unit") -> VlaDesc:
    if len(shape) == 4:
        B, H, T, d = shape
    elif len(shape) == 3:
        (B, T, d), H = shape, 1
    else:
        raise ValueError("inputs must be [B, H, T, d] or [N, T, d]")
    if dtype not in DTYPES:
        raise TypeError("dtype must be torch.float32 or torch.bfloat16")
    if path not in PATHS:
        raise ValueError(f"path must be one of {sorted(PATHS)}")
    if gain not in GAINS:
        raise ValueError(f"gain must be one of {sorted(GAINS)}")
    desc = VlaDesc(B=B, H=H, T=T, d=d, dtype=DTYPES[dtype], path=PATHS[path], eps=float(eps),
                   chunk=int(chunk), workspace=None, workspace_bytes=0, gain=GAINS[gain])
    if workspace is not None:
        if not (workspace.is_cuda and workspace.is_contiguous()):
            raise ValueError("workspace must be a contiguous device tensor")
        desc.workspace = workspace.data_ptr()
        desc.workspace_bytes = workspace.numel() * workspace.element_size()
    return desc


def _check(status: int, where: str):
    if status != 0:
        raise VlaError(status, where)


def workspace_size(shape, dtype, path="auto", chunk=0) -> int:
    lib = load_library()
    desc = make_desc(shape, dtype, path=path, chunk=chunk)
    n = ctypes.c_size_t(0)
    _check(lib.vla_workspace_size(ctypes.byref(desc), ctypes.byref(n)), "vla_workspace_size")
    return n.value


def resolve_path(shape, dtype, path="auto", chunk=0, gain="unit") -> str:
    lib = load_library()
    desc = make_desc(shape, dtype, path=path, chunk=chunk, gain=gain)
    p = ctypes.c_int32(0)
    _check(lib.vla_resolve_path(ctypes.byref(desc), ctypes.byref(p)), "vla_resolve_path")
    return {v: k for k, v in PATHS.items()}[p.value]


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, u: torch.Tensor,
            lambda0: float, eps: float = 1e-6, path: str = "auto", chunk: int = 0,
            return_state: bool = False, out: Optional[torch.Tensor] = None,
            S_final: Optional[torch.Tensor] = None, A_final: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None, stream: Optional[torch.cuda.Stream] = None):
    """VLA forward over [B, H, T, d] (or [N, T, d]) device tensors.

    Returns ``out`` (same shape and dtype as q), or ``(out, S_final, A_final)`` with the
    fp32 [.., d, d] final states when ``return_state`` is set or state buffers are given.
    """
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("u", u)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v, u must share shape, dtype and device")
    desc = make_desc(tuple(q.shape), q.dtype, eps=eps, path=path, chunk=chunk, workspace=workspace)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must match q in shape and dtype and be contiguous")
    state_shape = tuple(q.shape[:-2]) + (q.shape[-1], q.shape[-1])
    if return_state:
        if S_final is None:
            S_final = torch.empty(state_shape, dtype=torch.float32, device=q.device)
        if A_final is None:
            A_final = torch.empty(state_shape, dtype=torch.float32, device=q.device)
    for t in (S_final, A_final):
        if t is not None and (tuple(t.shape) != state_shape or t.dtype != torch.float32
                              or not t.is_contiguous()):
            raise ValueError("S_final / A_final must be contiguous fp32 [.., d, d]")
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        status = lib.vla_forward(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), u.data_ptr(), float(lambda0),
            out.data_ptr(),
            S_final.data_ptr() if S_final is not None else None,
            A_final.data_ptr() if A_final is not None else None,
            ctypes.byref(desc), s.cuda_stream)
    _check(status, "vla_forward")
    if S_final is not None or A_final is not None:
        return out, S_final, A_final
    return out


def _overlap(a: torch.Tensor, b: torch.Tensor) -> bool:
    """Whether two contiguous tensors share any byte of memory."""
    if a.device != b.device:
        return False
    a0, b0 = a.data_ptr(), b.data_ptr()
    return a0 < b0 + b.numel() * b.element_size() and b0 < a0 + a.numel() * a.element_size()


def forward_state(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, u: torch.Tensor,
                  lambda0: float = 1.0, S0: Optional[torch.Tensor] = None,
                  A0: Optional[torch.Tensor] = None, n0: Optional[torch.Tensor] = None,
                  eps: float = 1e-6, path: str = "auto", chunk: int = 0,
                  out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  stream: Optional[torch.cuda.Stream] = None,
                  S_final: Optional[torch.Tensor] = None, A_final: Optional[torch.Tensor] = None,
                  n_final: Optional[torch.Tensor] = None, gain: str = "unit",
                  noalloc: bool = False):
    """VLA forward continuing from a carried state (vla_forward_state in vla.h).

    S0 and A0 are fp32 [.., d, d] and n0 fp32 [.., d] device tensors, or None for the fixed
    start (S = 0, A = I / lambda0, n = 0); lambda0 is only used when A0 is None.  Returns
    (out, S_T, A_T, n_T), which a next call takes as its (S0, A0, n0); S_final, A_final and
    n_final optionally give the buffers to write them to (they must not be S0, A0, n0).
    ``gain="raw"`` runs the un-normalised-gain ablation (sequential and decode paths only).
    ``noalloc=True`` calls vla_forward_state_noalloc instead: the library allocates no device
    memory (the chunked path's scratch is its static per-GPU array; ``workspace`` must be None).
    """
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("u", u)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v, u must share shape, dtype and device")
    desc = make_desc(tuple(q.shape), q.dtype, eps=eps, path=path, chunk=chunk, workspace=workspace,
                     gain=gain)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must match q in shape and dtype and be contiguous")
    d = q.shape[-1]
    mat_shape = tuple(q.shape[:-2]) + (d, d)
    vec_shape = tuple(q.shape[:-2]) + (d,)
    for name, t, shp in (("S0", S0, mat_shape), ("A0", A0, mat_shape), ("n0", n0, vec_shape)):
        if t is not None and (tuple(t.shape) != shp or t.dtype != torch.float32 or not t.is_contiguous()
                              or t.device != q.device):
            raise ValueError(f"{name} must be a contiguous fp32 {shp} tensor on q's device")
    def _final(t, shp, name):
        if t is None:
            return torch.empty(shp, dtype=torch.float32, device=q.device)
        if tuple(t.shape) != shp or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous fp32 {shp} tensor")
        return t
    S_T = _final(S_final, mat_shape, "S_final")
    A_T = _final(A_final, mat_shape, "A_final")
    n_T = _final(n_final, vec_shape, "n_final")
    for a_name, a in (("S_final", S_T), ("A_final", A_T), ("n_final", n_T)):
        for b_name, b in (("S0", S0), ("A0", A0), ("n0", n0)):
            if b is not None and _overlap(a, b):
                raise ValueError(f"{a_name} overlaps {b_name}: the state is not updated in place")
    ptr = lambda t: t.data_ptr() if t is not None else None
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    fn = lib.vla_forward_state_noalloc if noalloc else lib.vla_forward_state
    with torch.cuda.device(q.device):
        status = fn(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), u.data_ptr(), float(lambda0),
            ptr(S0), ptr(A0), ptr(n0), out.data_ptr(), S_T.data_ptr(), A_T.data_ptr(),
            n_T.data_ptr(), ctypes.byref(desc), s.cuda_stream)
    _check(status, "vla_forward_state_noalloc" if noalloc else "vla_forward_state")
    return out, S_T, A_T, n_T


def la_workspace_size(shape, dtype) -> int:
    """Device workspace bytes of vla_linear_attention for [B, H, T, d] inputs."""
    lib = load_library()
    desc = make_desc(shape, dtype)
    n = ctypes.c_size_t(0)
    _check(lib.vla_la_workspace_size(ctypes.byref(desc), ctypes.byref(n)), "vla_la_workspace_size")
    return n.value


def linear_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, eps: float = 1e-6,
                     out: Optional[torch.Tensor] = None, S_final: Optional[torch.Tensor] = None,
                     n_final: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None,
                     stream: Optional[torch.cuda.Stream] = None):
    """Linear-attention baseline (vla_linear_attention in vla.h) over [B, H, T, d] (or
    [N, T, d]) device tensors.  Returns (out, S_T [.., d, d] fp32, n_T [.., d] fp32)."""
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v must share shape, dtype and device")
    desc = make_desc(tuple(q.shape), q.dtype, eps=eps, workspace=workspace)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must match q in shape and dtype and be contiguous")
    d = q.shape[-1]
    mat_shape = tuple(q.shape[:-2]) + (d, d)
    vec_shape = tuple(q.shape[:-2]) + (d,)
    for name, t, shp in (("S_final", S_final, mat_shape), ("n_final", n_final, vec_shape)):
        if t is not None and (tuple(t.shape) != shp or t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous fp32 {shp} tensor")
    if S_final is None:
        S_final = torch.empty(mat_shape, dtype=torch.float32, device=q.device)
    if n_final is None:
        n_final = torch.empty(vec_shape, dtype=torch.float32, device=q.device)
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        status = lib.vla_linear_attention(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                          S_final.data_ptr(), n_final.data_ptr(), ctypes.byref(desc),
                                          s.cuda_stream)
    _check(status, "vla_linear_attention")
    return out, S_final, n_final


def backward_workspace_size(shape, dtype, path="auto", chunk=0) -> int:
    """Device workspace bytes of vla_backward for [B, H, T, d] inputs."""
    lib = load_library()
    desc = make_desc(shape, dtype, path=path, chunk=chunk)
    n = ctypes.c_size_t(0)
    _check(lib.vla_backward_workspace_size(ctypes.byref(desc), ctypes.byref(n)),
           "vla_backward_workspace_size")
    return n.value


def backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, u: torch.Tensor, lambda0: float,
             d_out: torch.Tensor, dS_T: Optional[torch.Tensor] = None,
             dA_T: Optional[torch.Tensor] = None, dn_T: Optional[torch.Tensor] = None,
             eps: float = 1e-6, workspace: Optional[torch.Tensor] = None,
             stream: Optional[torch.cuda.Stream] = None, path: str = "auto", chunk: int = 0):
    """Gradients of <d_out, out> + <dS_T, S_T> + <dA_T, A_T> + <dn_T, n_T> through the
    forward from the fixed start (vla_backward in vla.h).  path "seq" runs one segment per
    stream, "chunk" the chunked path's time segments in parallel, "auto" picks.  Returns
    (dq, dk, dv, du) as fp32 tensors shaped like q and dlambda0, the per-stream shares [.., ] of
    dL/dlambda0."""
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("u", u), ("d_out", d_out)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v, u, d_out must share shape, dtype and device")
    d = q.shape[-1]
    mat_shape = tuple(q.shape[:-2]) + (d, d)
    vec_shape = tuple(q.shape[:-2]) + (d,)
    for name, t, shp in (("dS_T", dS_T, mat_shape), ("dA_T", dA_T, mat_shape), ("dn_T", dn_T, vec_shape)):
        if t is not None and (tuple(t.shape) != shp or t.dtype != torch.float32 or not t.is_contiguous()
                              or t.device != q.device):
            raise ValueError(f"{name} must be a contiguous fp32 {shp} tensor on q's device")
    desc = make_desc(tuple(q.shape), q.dtype, eps=eps, workspace=workspace, path=path, chunk=chunk)
    grads = [torch.empty(q.shape, dtype=torch.float32, device=q.device) for _ in range(4)]
    dlam = torch.empty(tuple(q.shape[:-2]), dtype=torch.float32, device=q.device)
    ptr = lambda t: t.data_ptr() if t is not None else None
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        status = lib.vla_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), u.data_ptr(), float(lambda0),
                                  d_out.data_ptr(), ptr(dS_T), ptr(dA_T), ptr(dn_T),
                                  *(g.data_ptr() for g in grads), dlam.data_ptr(), ctypes.byref(desc),
                                  s.cuda_stream)
    _check(status, "vla_backward")
    return (*grads, dlam)


def profile_enable(on: bool = True) -> None:
    """Record a HIP event pair around every kernel the library launches (see vla.h)."""
    _check(load_library().vla_profile_enable(1 if on else 0), "vla_profile_enable")


def profile_reset() -> None:
    _check(load_library().vla_profile_reset(), "vla_profile_reset")


def profile_read() -> dict:
    """{kernel name: (total milliseconds, launches)}; waits for the recorded events."""
    lib = load_library()
    n = lib.vla_profile_count()
    res = {}
    buf = ctypes.create_string_buffer(128)
    for i in range(n):
        ms = ctypes.c_double(0)
        cnt = ctypes.c_int64(0)
        _check(lib.vla_profile_get(i, buf, 128, ctypes.byref(ms), ctypes.byref(cnt)),
               "vla_profile_get")
        res[buf.value.decode()] = (ms.value, cnt.value)
    return res
