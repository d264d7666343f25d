"""Fused MoE-LoRA layer for MI355X (gfx950)."""
