"""CPU oracle of the W4A4 quantized linear layer (test infrastructure only)."""
