"""MI355X-native exact ring-attention forward.

The hot path lives in librattn.so (hand-written HIP for gfx950, C ABI in
include/rattn.h).  This package only marshals arguments to it:

    from ring_attention_amd import fwd, fwd_step, merge
    out, lse = fwd(q, k, v, causal=True, n_ring_steps=8, zigzag=True, rank=2)

Importing the package does not load the library; the first call does, and
raises if it has not been built (python -m ring_attention_amd.build).
"""
from __future__ import annotations

__all__ = ["fwd", "fwd_step", "merge", "status_string", "load_library"]


def __getattr__(name):
    if name in __all__ or name in ("RattnError", "LIB_PATH", "EXPORTS", "DTYPE_CODES"):
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
