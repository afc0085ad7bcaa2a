"""Seeded synthetic input generators (random draws and dtype casts only)."""
