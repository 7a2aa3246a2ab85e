"""Seeded, chunk-addressable synthetic inputs for the OSCAR INT2 KV-cache path.

This module only draws random numbers and rounds them to the input dtype
(bf16, round-to-nearest-even from fp32).  It holds none of the method's
arithmetic (no rotation, no quantisation, no attention), so both the CPU
oracle and the GPU path may consume what it produces.
"""
from .gen import *  # noqa: F401,F403
