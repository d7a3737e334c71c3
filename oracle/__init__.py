"""CPU oracle for the QoQ W4A8 GEMM path (test infrastructure only).

This package is the plain, slow, obviously-correct reference that the HIP
library is checked against.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it; the library never does, and it
never imports the library.
"""

from .qoq_oracle import *  # noqa: F401,F403
from .qoq_oracle import __all__  # noqa: F401
