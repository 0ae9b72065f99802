"""SCAPE's per-step sparse optimizer path for MI355X (gfx950).

The compute lives in ``libscape.so`` (hand-written HIP behind a C ABI, declared
in ``include/scape.h``).  ``sparse_communication_distributed_amd.scape`` is the
thin ctypes binding; ``workload`` builds layouts and seeded inputs.  Importing
the package loads nothing; the binding loads the library on first use and
raises if it is missing.
"""

__all__ = ["workload", "scape"]
