"""Hadamard-rotated 1-bit GEMV/GEMM for AMD MI355X (gfx950).

The computation runs in libpq1.so (HIP kernels behind the C ABI declared in
include/pq1.h); ``gemm_hadamard_rotated_amd.pq1`` is its Python binding and
``gemm_hadamard_rotated_amd.workloads`` draws the seeded synthetic inputs.
"""

__all__ = ["pq1", "workloads"]
