"""Seeded synthetic workloads (inputs only; no verification arithmetic)."""
