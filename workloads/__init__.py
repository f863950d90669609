"""Seeded synthetic workloads for tile-sparse video attention (inputs only)."""
from .configs import WORKLOADS, HEADLINE, Workload  # noqa: F401
