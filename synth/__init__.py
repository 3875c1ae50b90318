"""Seeded synthetic inputs for the OSCAR INT2 KV path.

This package draws random numbers and lays them out in the buffers the
library and the oracle both consume.  It holds none of the method's
arithmetic (no rotation, no quantization, no attention): every function here
either samples a distribution, rounds a sample to bf16 storage, or builds an
index table.
"""
from .workloads import *  # noqa: F401,F403
