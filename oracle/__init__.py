"""fp64 CPU oracle for the VLA forward recurrence and its linear-attention baseline
(test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this package.  The product path (``rls_associative_memory_amd``) never does.
"""

from .vla_oracle import init_state, phi, vla_forward, vla_step  # noqa: F401
from .la_oracle import la_forward  # noqa: F401
from .vla_grad import vla_forward_torch, vla_grad  # noqa: F401
