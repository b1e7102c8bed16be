"""Compressed PagedAttention hot path for MI355X (gfx950).

The compute lives in ``libzp.so`` (hand-written HIP kernels behind the C ABI
of ``include/zp.h``); this package only loads it and marshals arguments.
"""
from ._binding import (  # noqa: F401
    ZP_BF16, ZP_ERR_HIP, ZP_ERR_INVALID, ZP_ERR_NO_BLOCKS, ZP_ERR_STATE, ZP_F32, ZP_OK,
    BlockPool, KVCache, PrefixIndex, Scheduler, ZpError, append_kv, compress, compress_plan,
    compress_query, compress_workspace_bytes,
    last_error, lib, paged_decode, paged_decode_noalloc, paged_decode_workspace_bytes, profile_enable, profile_read,
    redundancy_all, ZP_DEBUG_POISON, ZP_DEBUG_TRACE, ZP_DEBUG_VALIDATE, debug_flags,
    set_debug_flags, trace_available,
)
