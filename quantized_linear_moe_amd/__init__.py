"""quantized_linear_moe_amd: the Quant Experts (QE) linear-layer hot path on MI355X.

The compute lives in libqe.so (hand-written HIP for gfx950, C ABI in include/qe.h);
this package is its ctypes binding plus a small holder for prepared layers.
Importing it fails if the shared library has not been built.
"""

from . import _libqe as libqe  # noqa: F401  (raises ImportError when libqe.so is missing)
from ._libqe import QEError, make_linear, qe_linear  # noqa: F401
from .linear import QELinear  # noqa: F401

__all__ = ["libqe", "QEError", "QELinear", "make_linear", "qe_linear"]
