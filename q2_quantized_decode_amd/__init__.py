"""Q2_K quantised decode for AMD MI355X (gfx950)."""
