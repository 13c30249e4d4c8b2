"""Seeded synthetic workloads (inputs only) shared by the tests, the benchmark and the smoke check."""
from .inputs import *  # noqa: F401,F403
from .inputs import __all__  # noqa: F401
