"""Seeded synthetic workloads shared by the oracle and the GPU tests/bench."""
