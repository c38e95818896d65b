"""Seeded synthetic workloads shared by tests and bench.py.

This package only draws random inputs with the shapes and distributions of
the DiffKV workloads; it contains none of the method's arithmetic
(classification, quantization, allocation, attention).
"""
from .synth import CONFIGS, config, make_prompt, make_decode, probe_queries, zipf_scores  # noqa: F401
