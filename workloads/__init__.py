"""Seeded synthetic workloads (shapes, seeds and input generators) for the
Engram layer forward. Shared by the tests, the benchmark and the smoke check;
holds none of the layer's arithmetic."""
from .configs import WORKLOADS, C0, C1, C2, C3, C4, EngramWorkload, ROW_F32, ROW_E4M3_E8M0  # noqa: F401
from . import gen  # noqa: F401
