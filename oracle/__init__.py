"""CPU oracle for the canvas denoising step (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg import this
package.  It shares no code with the HIP library.
"""
from . import dg_oracle, fp8, philox  # noqa: F401
from .dg_oracle import *  # noqa: F401,F403
