"""KDA (Kimi Delta Attention) forward recurrence for AMD MI355X (gfx950)."""
