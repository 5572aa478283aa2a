"""Seeded synthetic inputs shared by the CPU oracle tests and the HIP path.

This package holds only input generation (random tensors of the shapes and
value distributions of the workloads) and no step of the compression method.
Both sides receive the same arrays from here; neither side imports the other.
"""
from .inputs import *  # noqa: F401,F403
