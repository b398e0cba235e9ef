"""libspecverify: the speculative-decoding verify step on MI355X (gfx950)."""
