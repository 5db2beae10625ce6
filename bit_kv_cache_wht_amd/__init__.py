"""UltraQuant FP4 KV-cache hot path for MI355X (gfx950): Python binding."""
