"""Layerwise QK-Norm for AMD Instinct MI355X (gfx950)."""
