"""CPU oracle of the block-discrete-diffusion canvas step.

Test infrastructure: only tests/, the smoke check and the benchmark's
CPU-baseline leg import this package.  It shares no code with the HIP library.
"""
from .dg_oracle import *  # noqa: F401,F403
