"""Seeded synthetic inputs shared by the tests, the bench and the smoke check."""
from .gen import (  # noqa: F401
    CONFIGS, DESCRIPTIONS, Workload, WriteCall, config, make_workload, prefill_queries,
)
