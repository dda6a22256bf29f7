"""CPU oracle for the ResidualKV hot path -- test infrastructure only.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg
may import this package.  It shares no code with the HIP library.
"""

from .rkv_oracle import *  # noqa: F401,F403
