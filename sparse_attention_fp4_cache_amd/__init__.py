"""CSA2 sparse attention over an FP4 global KV cache, for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libcsa2fp4.so`` (hand-written HIP
kernels, declared in ``include/csa2fp4.h``); ``lib`` is a thin ctypes binding
with the same entry-point names, ``step`` composes the Full / Reindex / Reuse
layer modes from those calls, and ``workloads`` draws seeded synthetic inputs.
Importing this package loads nothing; the library is opened on first use.
"""
__all__ = ["lib", "step", "workloads"]
