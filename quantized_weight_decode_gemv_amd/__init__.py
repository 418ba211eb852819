"""qwg: fused dequantize + GEMV over block-quantized weights (Q4_K, IQ3) for MI355X."""
