"""MI355X-native paged KV cache: slot-mapping scatter and paged decode read.

The compute lives in ``libpkv.so`` (hand-written HIP kernels for gfx950 behind a
C ABI declared in ``include/pkv.h``); this package is a thin ctypes binding that
marshals torch tensors into pointers and a HIP stream.  The library is loaded
on first use, and a missing library is an error: there is no fallback path.
"""
from .binding import (  # noqa: F401
    BlockAllocator, KVCacheExhausted, PkvError, ReadCounters, decode_step, library_path, load_library,
    paged_attention, paged_attention_into, paged_attention_multi, paged_attention_noalloc, read_tile,
    reshape_and_cache, workspace_size, workspace_size_multi,
)
