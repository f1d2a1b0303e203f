"""Plain CPU oracle for the fused quantized linear layer (test infrastructure only)."""
