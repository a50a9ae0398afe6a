"""Weight-only block-32 int4/int8 matmul for MI355X (gfx950)."""
