"""fp64 CPU oracle for query-oriented sparse KV selection and attention over
the selected keys.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are its only callers.  The HIP library never imports it, and it
imports nothing from the HIP library.  Every function is pinned by the CPU tests
against closed forms, invariants, brute force and hand-derived fixtures.
"""
from .quoka import *  # noqa: F401,F403
from . import quoka  # noqa: F401
