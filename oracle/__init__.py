"""CPU oracle for the ZeRO mixed-precision optimizer step.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
bench's CPU-baseline leg, never by the library. It shares no code with the
HIP path. See zero_step.py for the definitions and their page citations.
"""

from .zero_step import *  # noqa: F401,F403
from .zero_step import (  # noqa: F401
    ScalerState, AdamW, FP16, BF16, FP32, COPY, OVERWRITE, ACCUMULATE,
)
