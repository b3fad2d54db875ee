"""CPU oracle for the single-GPU MoE layer forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this package: only the test suite, the smoke check of the package entry point
and the benchmark's CPU-baseline leg use it.  It shares no code with the HIP
path (no kernels, headers, helpers, tables or pre/post-processing); the only
common dependency is the seeded input generator in ``workloads``.

The oracle is a plain, slow, staged NumPy implementation in float64.  bf16
inputs are widened exactly (the 16 stored bits become the top half of a binary32),
and no intermediate value is rounded.  Each function cites the passage it
follows.  See ``oracle.moe`` for the functions.

Parity pins: every function here is pinned by the ``-m "not gpu"`` tests
(brute force on tiny inputs, closed forms, invariants, textbook special cases,
the printed vectors of the ep_dispatch.rs tests and the w13 byte-offset check of
the modelexpress refit test).  No function is "parity unpinned".
"""
from .moe import *  # noqa: F401,F403
from .moe import __all__  # noqa: F401
