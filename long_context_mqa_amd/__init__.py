"""HySparse2 attention hot path on MI355X: the Python binding of libhs2.

The compute runs in hand-written HIP kernels for gfx950 behind the C ABI declared in
include/hs2.h; this package only marshals arguments (see hs2.py).
"""
from .hs2 import (  # noqa: F401
    Batch,
    HS2Error,
    bridge_kv,
    bridge_kv_workspace_size,
    full_attn_select,
    full_attn_select_workspace_size,
    load,
    sparse_attn,
    sparse_attn_workspace_size,
)
