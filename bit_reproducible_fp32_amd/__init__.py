"""Reproducible fixed-order FP32 matmul for MI355X (gfx950)."""
