"""CPU fp64 oracle for CCA attention -- test infrastructure only.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg
import this package.  It shares no code with the HIP library.
"""
from .cca_oracle import *  # noqa: F401,F403
from .cca_oracle import __all__  # noqa: F401
