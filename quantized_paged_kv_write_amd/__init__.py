"""kvq: quantized paged KV cache for MI355X (gfx950).

The HIP library (csrc/, built into libkvq.so) quantizes K/V on write into a
paged cache and runs dequantizing paged decode and causal chunked-prefill
attention; `binding` exposes
its C ABI to torch tensors and `workloads` draws seeded synthetic inputs.
"""
from .binding import (COPY_NARROW_WORKGROUPS, DEVERR, DTYPES, CopyCall, DecodeCall, KvqError, PagedKVCache, copy_blocks, decode_attn,  # noqa: F401
                      decode_attn_noalloc, decode_workspace_bytes, get_device_error, lib, prefill_attn,
                      prefill_workspace_bytes, status_string, write, write_static)
