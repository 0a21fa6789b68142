"""fp64 CPU reference oracle for the selective scan -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never calls it and has
no fallback to it.  See ``ssm_oracle.c`` for the passages it follows.

Every function here has a pin in ``tests/test_oracle_pins.py`` (closed forms,
the matrix-exponential ZOH identity, the LTI convolution mode, limits and
invariants; for the backward, finite differences of the forward and exact
adjoint dot-product identities); no function is "parity unpinned".
"""
from .oracle import (Oracle, scan, scan_bwd, scan_complex, scan_complex_bwd, scan_ssd, step,  # noqa: F401
                     step_complex, max_threads, load)
