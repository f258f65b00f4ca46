"""Head-wise sparse decode attention on AMD MI355X (gfx950).

The compute lives in ``libhws.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/hws.h``).  ``head_wise_sparse_02_amd.hws`` is a thin
ctypes binding with the same call names; ``workloads`` builds seeded
synthetic inputs.  Importing this package loads nothing: the library is
opened on first use and a missing library raises at that point.
"""

__all__ = ["hws", "workloads"]
