"""Causal structured-sparse attention for MI355X (gfx950).

The compute path is the HIP library ``libsparse_attn.so`` (C ABI declared in
``include/sparse_attn.h``).  This package is a thin binding over it: argument
checks and marshalling only.  ``inputs`` holds the seeded synthetic workloads.
The library is loaded on first use, not at import time.
"""
from .binding import (MODE_ECP, MODE_PI, MODE_WINDOW, SparseAttnError, attention, bwd,
                      bwd_workspace_size, decode, decode_noalloc, decode_paged, decode_ring,
                      decode_workspace_size, fwd,
                      fwd_workspace_size, library_path, load_library, loop_fwd)

__all__ = ["fwd", "bwd", "attention", "decode", "decode_noalloc", "decode_ring", "decode_paged", "loop_fwd", "fwd_workspace_size", "bwd_workspace_size",
           "decode_workspace_size",
           "load_library", "library_path", "SparseAttnError", "MODE_PI", "MODE_WINDOW",
           "MODE_ECP"]
