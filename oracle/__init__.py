"""CPU oracle for the OSCAR INT2 KV-cache hot path (test infrastructure only:
imported by tests, the smoke entry point and the benchmark's CPU-baseline leg;
never by the product path)."""
from .oscar_ref import *  # noqa: F401,F403
