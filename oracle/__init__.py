"""CPU oracle for the heterogeneous-batch forward step — TEST INFRASTRUCTURE.

This package is a plain, slow, obviously correct numpy implementation of
what one step of the heterogeneous-batch runner computes, written from the
page "Efficient Iterative Retrieval with Heterogeneous Batching" (paperpeel
full text, §3 Unified Runner: §3.1 High-Level Workflow, §3.2 Batch Unit,
§3.3 Incremental Pooler) and its summary page (agihunt, the paragraphs on
the three batch units and on incremental pooling).  It computes in fp32 by
default and in fp64 when asked (pinning mode).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The product path (the HIP library and its
binding) never imports, links or calls anything here, and this package
shares no code with it; the two meet only through the seeded input
generators in ``synth/``.

Functions whose result is not fixed by any pin are marked "parity unpinned"
in their docstrings.  Every other function is pinned by ``tests/oracle``.
"""

from .pack import pack_py, PackError, OK, EINVAL, ENOPAGES, ECAPACITY, ESTATE
from .forward import (rmsnorm, rope, silu, attend_item, layer, step, StepOut,
                      widen_weights, new_pool, new_kv)
from .pooling import pool_item

__all__ = ["pack_py", "PackError", "OK", "EINVAL", "ENOPAGES", "ECAPACITY", "ESTATE",
           "rmsnorm", "rope", "silu", "attend_item", "layer", "step", "StepOut", "widen_weights",
           "new_pool", "new_kv", "pool_item"]
