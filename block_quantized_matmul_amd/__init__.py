"""Block-quantized MUL_MAT (GGUF Q4_0 / Q8_0) for the AMD MI355X (gfx950)."""
