"""fp64 CPU oracle for the exact attention forward pass.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product library.

``oracle.py`` is the plain definition (C, fp64).  ``tiled.py`` restates the
pages' tile-by-tile algorithms in numpy fp64; it exists only to pin the
definition and the pages' claim that tiling leaves the result unchanged.
"""
from .oracle import Oracle, build, default  # noqa: F401
