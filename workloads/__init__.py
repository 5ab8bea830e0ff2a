"""Seeded synthetic workloads (shapes, hyperparameters, random draws)."""
