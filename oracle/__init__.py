"""fp64 CPU oracle of the SparsePR attention call.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the
bench's CPU-baseline leg import this package; the product path never does.
"""
from . import brute
from .sparsepr_oracle import *  # noqa: F401,F403
