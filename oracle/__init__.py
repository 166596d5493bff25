"""Plain, slow, fp64 CPU oracle for query-aware block-sparse attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import this package.  It shares no code with the HIP
library and imports nothing from it; the library never calls it.
"""
from .bsa_oracle import *  # noqa: F401,F403
