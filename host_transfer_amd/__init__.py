"""Invariant Bit Packing (IBP) gather + decompress for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library libibp.so (HIP kernels, declared in
include/ibp.h); `host_transfer_amd.ibp` is its thin ctypes binding and
`host_transfer_amd.workloads` draws the seeded synthetic inputs.  Importing
this package loads nothing: the library is loaded by the binding on first use.
"""
__all__ = ["ibp", "workloads"]
