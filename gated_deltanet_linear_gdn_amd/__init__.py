"""Gated delta-rule decode and chunked prefill on MI355X (gfx950)."""
