"""CPU oracle for the Mixture-of-Recursions forward pass (test infrastructure only).

This package is the plain, slow reference the HIP library is checked against.
Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
it; the library never calls it and it never calls the library.

See ``oracle/mor.py`` for the method itself. Parity status per function is
listed in the module docstring there.
"""
from .mor import *  # noqa: F401,F403
