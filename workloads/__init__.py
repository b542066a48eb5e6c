"""Seeded synthetic workloads shared by the tests, the bench and smoke()."""
from .synth import ALL, DIT480, DIT720, LLM8K, LLM128K, TINY, Workload, make_inputs, small  # noqa: F401
