"""Seeded synthetic inputs shared by the tests, the smoke check and the
benchmark.  Holds no part of the attention method's arithmetic."""
from . import gen, workloads  # noqa: F401
from .workloads import WORKLOADS, Workload, custom  # noqa: F401
