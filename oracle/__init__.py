"""CPU oracle for block-scaled FP4 quantize / dequantize (test infrastructure only)."""
