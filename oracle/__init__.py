"""CPU oracle for the compressed sparse attention layer.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product package never does.
"""
from .oracle import *  # noqa: F401,F403
