"""ART-terminated decode attention for MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of
include/art.h (libart.so, built in-tree).  This package only marshals
arguments (see _binding.py); it never computes attention itself.
"""
from ._binding import (ART_BF16, ART_F32, ART_I4, ART_I8, EXPORTS, LIB_PATH, ORDER_ASCENDING, ORDER_LIST,
                       ORDER_RECENT, ArtDesc, ArtError, decode_attention, load, make_desc, validate,
                       workspace_bytes)

__all__ = ["decode_attention", "workspace_bytes", "validate", "make_desc", "load", "ArtDesc",
           "ArtError", "ART_F32", "ART_BF16", "ART_I8", "ART_I4", "EXPORTS", "LIB_PATH", "ORDER_ASCENDING",
           "ORDER_RECENT", "ORDER_LIST"]
