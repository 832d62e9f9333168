"""Seeded synthetic inputs shared by the oracle-side tests and the HIP path.

This package draws random numbers and lays them out; it performs none of the
method's arithmetic (no rotation of cache entries, no quantisation, no packing,
no attention).  See ``synth.inputs``.
"""
from .inputs import *  # noqa: F401,F403
