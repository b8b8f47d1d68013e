"""MI355X (gfx950) dense GEMM library: Python binding over the C ABI."""
