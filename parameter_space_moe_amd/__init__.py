"""Swimba (Switch Mamba) parameter-space-MoE selective scan for MI355X (gfx950)."""
