"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke run.

This package generates data only: weights, activations, logits, token
histories, draft candidates and uniform random draws.  It holds none of the
verify step's arithmetic, so the oracle and the GPU library can both be fed
from it without sharing any of the method's code.
"""

from .inputs import *  # noqa: F401,F403
