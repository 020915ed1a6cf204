"""Sliding Tile Attention forward for AMD MI355X (gfx950)."""
