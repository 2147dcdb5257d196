"""CPU oracle for the DFlash draft step (test infrastructure only).

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import it.
The GPU library shares no code with it and never calls it."""
from .dflash_oracle import *  # noqa: F401,F403
from . import dflash_oracle as ref  # noqa: F401
