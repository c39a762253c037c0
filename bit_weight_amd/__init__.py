"""Sherry 3:4-sparse ternary matmul for MI355X (gfx950)."""
