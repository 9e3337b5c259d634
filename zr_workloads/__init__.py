"""Synthetic workloads and seeded input generators shared by tests, smoke check
and benchmark.  Data definitions only: no partitioning, reduction or update
arithmetic lives here."""
from .configs import ALL, BY_NAME, FLAT_1T, FLAT_7B, GPT_7P5B, LLAMA_7B, TINY_MLP, Workload  # noqa: F401
