"""libswasink: hybrid sliding-window attention forward for MI355X (gfx950)."""
