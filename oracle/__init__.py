"""CPU oracle for MLA decode (test infrastructure only; see mla_oracle.py).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The HIP library never does.
"""
from . import mla_oracle  # noqa: F401
