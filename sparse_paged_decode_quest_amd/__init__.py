"""Sparse paged decode attention for AMD MI355X (gfx950).

The computation lives in the HIP library ``libspd.so`` behind the C ABI of
``include/spd.h``; ``_abi`` is its ctypes binding (same entry-point names), ``step``
allocates device buffers and calls the entry points in order, and ``workloads`` draws
seeded synthetic inputs.
"""
from . import workloads  # noqa: F401

__all__ = ["workloads"]
