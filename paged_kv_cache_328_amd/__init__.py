"""libpagedattn: paged decode attention for MI355X (gfx950).

The compute path is the C-ABI shared library libpagedattn.so built from
csrc/ (hand-written HIP kernels plus the host block allocator); the Python
module `pagedattn` is a thin ctypes binding over it.  `workloads` draws the
seeded synthetic inputs.
"""
