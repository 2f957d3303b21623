"""Paged KV-cache attention for AMD Instinct MI355X (gfx950).

The hot path of PagedAttention — slot scatter, paged decode (with split-KV
partitions and a grouped-query matrix-core variant), causal chunked prefill
and copy-on-write block copies — as hand-written HIP kernels behind the C ABI
of ``libpkv.so`` (``include/pkv.h``).  This package is the thin Python
binding over that library (ctypes + torch device memory and streams), plus
the host-side block manager and the seeded synthetic workloads.
"""
from ._binding import (PARTITION_AUTO, PagedKVCache, PkvError, copy_blocks, decode_workspace_bytes,
                       gather_kv, lib, paged_decode, paged_decode_append, paged_decode_noalloc,
                       paged_mixed, paged_prefill, reshape_and_cache, validate_host, version)

__all__ = ["PARTITION_AUTO", "PagedKVCache", "PkvError", "copy_blocks", "decode_workspace_bytes",
           "gather_kv", "lib", "paged_decode", "paged_decode_append", "paged_decode_noalloc",
           "paged_mixed",
           "paged_prefill", "reshape_and_cache", "validate_host", "version"]
