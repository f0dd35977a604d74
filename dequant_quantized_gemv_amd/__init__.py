"""ggml block-quantized dequantize / GEMV / GEMM on gfx950 (MI355X)."""
