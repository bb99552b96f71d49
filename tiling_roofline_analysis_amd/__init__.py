"""MI355X-native single-precision GEMM (C = A x B, row-major) for gfx950."""
