"""Hadamard-rotated 1-bit GEMV/GEMM for AMD MI355X (gfx950)."""
