"""MI355X-native OSCAR split-cache INT2 decode attention.

The compute path is liboscar.so (HIP kernels for gfx950, C ABI in
include/oscar.h); ``binding`` is its thin ctypes wrapper and ``splitcache``
holds the host-side bookkeeping of page tables and the recent-window ring.
"""
from . import binding  # noqa: F401
from .binding import (Cache, DecodeArgs, OscarError, alloc_workspace, decode, decode_attn,  # noqa: F401
                      demote_pack, merge, record_bytes, workspace_bytes, write_bf16)

__all__ = ["binding", "Cache", "DecodeArgs", "OscarError", "alloc_workspace", "decode",
           "decode_attn", "demote_pack", "merge", "record_bytes", "workspace_bytes", "write_bf16"]
