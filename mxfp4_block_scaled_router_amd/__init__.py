"""MXFP4 routed-expert MoE layer for MI355X (gfx950)."""
