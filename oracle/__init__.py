"""Float64 CPU oracle for the EXL3 linear layer (test infrastructure only).

Only the test suite, the smoke check and the benchmark's cpu_baseline leg may
import this package.  The HIP path never imports it and shares no code with it.
"""
from .exl3_oracle import *  # noqa: F401,F403
