"""Paged KV-cache attention for MI355X (gfx950): placeholder, filled in below."""
