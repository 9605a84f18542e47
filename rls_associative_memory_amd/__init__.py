"""MI355X-native VLA forward recurrence.

The compute path is the C-ABI library ``librls_vla.so`` (hand-written gfx950 HIP kernels);
``rls_associative_memory_amd.vla`` is the thin ctypes binding that marshals torch device
tensors and the current HIP stream into it.  Importing this package loads nothing: the
library is opened on first use and a missing library is an error, never a fallback.
"""

__all__ = ["forward", "forward_state", "linear_attention", "workspace_size", "library_path", "VlaError"]


def __getattr__(name):
    if name in __all__:
        from . import vla
        return getattr(vla, name)
    raise AttributeError(name)
