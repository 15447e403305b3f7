"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This package draws random numbers and lays them out the way the paged cache
stores them.  It holds none of the attention arithmetic: no dot products, no
softmax, no projections, no rotation.  Both the CPU oracle and the GPU library
consume what it produces; neither is imported here.
"""
from .inputs import *  # noqa: F401,F403
from .configs import *  # noqa: F401,F403
