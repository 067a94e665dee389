"""Sliding-window attention for AMD MI355X (gfx950).

The compute lives in the HIP library ``libswa.so`` behind the C ABI declared in
``include/swa.h``; this package only marshals torch tensors into it (see
``binding.py``).  Importing the package does not load the library; the first
call does, and fails loudly if it has not been built.
"""
from .binding import (  # noqa: F401
    SwaError, fwd, fwd_workspace_size, fwd_cached, kv_append, kv_append_chunk, decode,
    decode_workspace_size, decode_sinks, decode_sinks_workspace_size, kv_append_paged,
    decode_paged, bwd, bwd_workspace_size, load_library,
)
