"""Seeded synthetic inputs shared by the tests, the bench and the oracle runs.

Holds none of the method's arithmetic: only shapes, hyper-parameters,
random numbers, needle planting and dtype casts.
"""
from .configs import CONFIGS, Config  # noqa: F401
from .inputs import make_inputs, needle_blocks, paged_cache, varlen_lengths  # noqa: F401
