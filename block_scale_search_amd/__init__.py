"""NVFP4 per-group E4M3 block-scale search on MI355X (gfx950)."""
