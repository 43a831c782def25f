"""Seeded synthetic inputs for the PLE n-gram embedding path.

This package is the only code that both the CPU oracle and the HIP path take
their inputs from. It holds none of the method's arithmetic (no n-gram hash,
no FP8 decode, no projection, gate or convolution): only token streams,
sequence boundaries, hidden states, weights and the FP8 table, each drawn
from a fixed seed.
"""

from .inputs import *  # noqa: F401,F403
