"""Seeded synthetic inputs shared by the tests, the bench and the smoke check."""
from .gen import CONFIGS, DESCRIPTIONS, Workload, WriteCall, config, make_workload  # noqa: F401
