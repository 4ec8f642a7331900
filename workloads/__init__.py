"""Synthetic workloads (shapes and seeded inputs) for the sharded-step tests and bench."""
