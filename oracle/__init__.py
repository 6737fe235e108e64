"""CPU oracle of the CSA2 hot path (NumPy, float64).

TEST INFRASTRUCTURE ONLY: the HIP library never imports, links or runs anything
here.  Only the tests, the smoke check and the CPU-baseline leg of the benchmark
use it.  ``codecs`` holds the number formats, ``csa2`` the method's steps.
"""
from . import codecs, csa2  # noqa: F401
