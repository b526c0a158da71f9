"""gated_delta_rule_63_amd: the gated-delta-rule state recurrence on MI355X (gfx950).

The compute lives in ``libgdr.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/gdr.h``).  This package holds the thin ctypes binding
(``gated_delta_rule_63_amd.gdr``), the build step and the seeded input
generators.  Importing the package does not load the library; the first call
through the binding does, and fails loudly if it has not been built.
"""
__all__ = ["gdr", "inputs"]
