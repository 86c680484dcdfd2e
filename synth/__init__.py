"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

Holds no arithmetic of the denoising method: only counter-based value
generation (``hashgen``) and workload geometry plus tensor recipes
(``workloads``).
"""
from . import hashgen, workloads  # noqa: F401
