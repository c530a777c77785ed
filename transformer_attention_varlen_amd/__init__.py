"""kattn: packed variable-length attention for the AMD MI355X (gfx950).

The compute path is the C-ABI library ``libkattn.so`` built from ``csrc/``
(hand-written HIP kernels).  ``kattn`` holds the thin ctypes binding with the
same names as the C entry points; ``workloads`` draws seeded synthetic inputs.
Importing this package does not load the library; the first call does, and it
raises if the library has not been built.
"""
