"""CPU oracle for the per-layer DP clip-and-accumulate step (float64, plain, slow).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package smoke check
and by the benchmark's CPU-baseline leg, never by the product path.  It shares
no code with the HIP library; the seeded input generators in ``workloads``
are the only module both sides use.

Pins (what checks this oracle against something other than itself) live in
``tests/test_oracle_pins.py``; every function here is pinned there.
"""
from . import philox  # noqa: F401
from .dp_linear import (  # noqa: F401
    oracle_linear, oracle_projected, oracle_norms, oracle_entries,
    brute_force_linear, widen, select_active, clip_factor, per_sample_grad,
)
