"""Seeded synthetic inputs shared by the oracle tests and the GPU path."""
from .workloads import *  # noqa: F401,F403
