"""fp64 CPU oracle for the Based layer -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package.  The product path never does.
"""

from .based_oracle import (  # noqa: F401
    D_K,
    D_PHI,
    DecodeState,
    linattn_chunked,
    linattn_quadratic,
    linattn_recurrent,
    linattn_state,
    phi,
    swa,
    taylor_kernel,
)
