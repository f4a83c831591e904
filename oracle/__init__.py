"""fp64 CPU oracle for the HSTU layer forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import anything from here.  The HIP library never calls it, links it or falls back
to it; it shares no code, helper or table with the library.

Modules:
  hstu_ref          vectorised float64 layer, attention, norm-gate and M-FALCON forward
  brute             scalar loop version of the layer for tiny inputs
  stochastic_length the Stochastic Length keep / subsample rule

Every function is pinned by ``-m "not gpu"`` tests against brute force, invariants,
closed forms and library cross-checks; none is marked "parity unpinned".
"""

from . import brute, hstu_ref, stochastic_length  # noqa: F401
