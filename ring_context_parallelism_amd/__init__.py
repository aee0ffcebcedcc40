"""Zigzag ring context-parallel attention for MI355X (gfx950).

The computation lives in ``libcpattn.so`` (HIP kernels behind the C ABI of
``include/cp_attn.h``); this package only marshals arguments to it.
"""

from .api import Plan, lse_merge  # noqa: F401
from ._native import CpAttnError  # noqa: F401

__all__ = ["Plan", "lse_merge", "CpAttnError"]
