"""Synthetic workloads (shapes, layout parameters) and seeded input generators."""
from .configs import Workload, ALL, BY_NAME  # noqa: F401
