"""libcpattn: context-parallel ring attention on MI355X (gfx950)."""
