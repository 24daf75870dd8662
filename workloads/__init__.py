"""Seeded synthetic workloads (inputs only) for the SMC-SD verify / resample path."""
from .configs import ALL, BY_NAME, C1, C2, C3, C4, C5, Config, downsized, get  # noqa: F401
