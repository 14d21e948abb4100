"""Lossless BF16 weight compression fused into the decode-time GEMM, for MI355X (gfx950)."""
