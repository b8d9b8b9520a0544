"""CPU oracle for the DFlash2 draft-block head (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The library never does.
"""
from . import dflash2_oracle  # noqa: F401
