"""Seeded synthetic inputs for the paged-attention path.

This package is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It only draws random numbers and lays them into the cache-pool
shapes; it holds none of the attention arithmetic, no gather and no softmax.
Neither ``oracle`` nor ``paged_kv_cache_185_amd`` is imported here.
"""
from .gen import *  # noqa: F401,F403
