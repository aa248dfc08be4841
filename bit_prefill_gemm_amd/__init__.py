"""MI355X-native Hadamard-rotated W4A4 prompt GEMM (placeholder; binding added next)."""
