"""Seeded synthetic input generators (no optimizer arithmetic)."""
