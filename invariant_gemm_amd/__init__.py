"""invariant_gemm_amd -- batch-invariant GEMMs for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libbigemm.so`` (hand-written HIP
kernels); ``invariant_gemm_amd.bigemm`` is its thin ctypes binding and
``invariant_gemm_amd.inputs`` the seeded generators and operand quantisers.
Importing this package loads neither, so CPU-only users (the quantisers)
do not need the HIP library.
"""

__all__ = ["bigemm", "inputs"]
