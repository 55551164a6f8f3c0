"""Reference oracle for exact scaled-dot-product attention, forward and backward.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain, fp64 CPU statement of
what the attention kernels compute.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  The product package
(``exact_attention_27_amd``) never imports it, shares no code with it, and fails
loudly when its HIP library is missing instead of falling back to anything here.

Every function here is pinned by ``tests/test_oracle.py`` to facts that do not
come from the oracle itself (closed forms, invariants, finite differences,
brute force, and an fp64 library cross-check).
"""

from .attention import (  # noqa: F401
    attention_backward,
    attention_forward,
    head_backward,
    head_forward,
    kv_head_of,
)
