"""CPU oracle of the DSA decode hot path — test infrastructure only.

Only tests, the smoke check and the benchmark's CPU-baseline leg may import this
package.  It shares no code with the HIP library.
"""
from .dsa_oracle import *  # noqa: F401,F403
