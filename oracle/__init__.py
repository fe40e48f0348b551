"""fp64 CPU oracle for the retention forward pass — TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. It shares no code with the HIP path and the HIP path never calls
it. Pinned by tests/test_oracle.py (brute force, closed forms, invariants,
library special cases); no function here is left unpinned.
"""
from .retention import *  # noqa: F401,F403
from .retention import __all__  # noqa: F401
