"""Seeded synthetic inputs shared by the oracle-side tests and the HIP path.

This package only draws random numbers and lays them out.  It holds none of
the arithmetic of the block-sparse attention method (no pooling, no softmax,
no mask rules, no permutation planning), so that the fp64 oracle and the HIP
library can both consume it without sharing any method code.
"""

from .configs import CONFIGS, Workload, get_config  # noqa: F401
from .synth import generate, p1_demo_inputs  # noqa: F401
