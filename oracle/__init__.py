"""CPU oracle for the MSA routing + sparse-attention path (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding)
never does.
"""
from .msa_oracle import *  # noqa: F401,F403
