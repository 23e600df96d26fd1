"""Paged decode attention for AMD MI355X (gfx950)."""
