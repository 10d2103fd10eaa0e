"""Seeded synthetic inputs shared by the HIP path's harness and the CPU oracle.

This package holds configuration records and random input generators only;
it computes no step of the denoising method.
"""
from . import configs, gen  # noqa: F401
from .configs import BY_ID, C1, C2, C3, C4, C5, ModelConfig, Workload  # noqa: F401
