"""Block-sparse tiled attention for AMD Instinct MI355X (gfx950)."""
