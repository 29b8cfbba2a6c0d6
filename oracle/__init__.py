"""fp64 CPU oracle for the approximate-attention prefill path (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
package. It shares no code with the HIP library and imports nothing from it.
"""
from .spava_oracle import *  # noqa: F401,F403
