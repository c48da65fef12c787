"""Ragged verify + acceptance for confidence-scheduled speculative decoding, on MI355X.

The product is the C-ABI library ``librva.so`` (HIP kernels for gfx950, declared in
``include/rva.h``); ``ragged_verify_acceptance_amd.rva`` is its thin Python binding.
"""

from . import rva  # noqa: F401
from .rva import RvaError  # noqa: F401

__all__ = ["rva", "RvaError"]
