"""Seeded synthetic inputs for the Quant Experts (QE) linear hot path.

This package only draws random tensors of the right shapes, dtypes and
structure.  It holds none of the method's arithmetic (no smoothing, no
quantization, no rounding rule of the method, no routing): both the CPU oracle
and the HIP library consume exactly the tensors produced here.

The activation structure follows what the pages observe about important
channels (Quant Experts paper, Figures 2 and 3 and the "Problem & Motivation"
section of the MCISLAB DeepRead summary): a few channels are large on nearly
every token, many others are large only on particular tokens, and the sets
differ between image and text tokens.
"""

from .configs import CONFIGS, LinearSpec, QEConfig, get_config  # noqa: F401
from .gen import (  # noqa: F401
    gen_activations,
    gen_linear,
    rng_for,
)
