"""MI355X (gfx950) fused exact attention: forward and backward with grouped-query
heads, bottom-right aligned causal / sliding-window masks, packed
variable-length batches, attention sinks, score variants and KV caches
(paged, in-place append, rotary embedding).

The compute path is libattn36.so (hand-written HIP kernels behind the C ABI in
include/attn.h); the functions here are its Python binding and have the same
names as the C entry points.
"""
from ._lib import (  # noqa: F401
    ATTN_BF16, ATTN_EHIP, ATTN_EINVAL, ATTN_ENOTSUP, ATTN_FP16, ATTN_FP32, ATTN_OK, AttnError,
    attn_bwd, attn_bwd_noalloc, attn_bwd_varlen, attn_fwd, attn_fwd_kvcache, attn_fwd_varlen, attn_kvcache_append, attn_rotary,
    attn_timing_enable, attn_timing_read, last_error, load_library, version,
)
