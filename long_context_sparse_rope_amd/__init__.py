"""MI355X (gfx950) sparse long-context prefill: DCA + YaRN RoPE +
vertical-slash sparse attention over a GQA KV cache.

The compute lives in liblcsr.so (HIP, C ABI in include/lcsr.h); this package
is its thin binding plus the chunk loop.  Importing it loads the library and
fails loudly if it has not been built.
"""

from . import _capi
from .ops import (LcsrError, RopeConfig, DcaConfig, Pattern, softmax_scale,
                  rope_yarn_apply, dca_positions, vs_pattern_estimate,
                  vs_sparse_attn_prefill, attn_decode, attn_decode_noalloc, attn_recall_check,
                  workspace_bytes,
                  pattern_fill_a_shape, BlockPattern, block_sparse_estimate,
                  block_sparse_attn_prefill, block_sparse_recall_check)
from .driver import ChunkedSparsePrefill, search_head_patterns

_capi.load()

__all__ = ["LcsrError", "RopeConfig", "DcaConfig", "Pattern", "softmax_scale",
           "rope_yarn_apply", "dca_positions", "vs_pattern_estimate",
           "vs_sparse_attn_prefill", "attn_decode", "attn_decode_noalloc", "attn_recall_check",
           "workspace_bytes",
           "pattern_fill_a_shape", "BlockPattern", "block_sparse_estimate",
           "block_sparse_attn_prefill", "block_sparse_recall_check", "ChunkedSparsePrefill",
           "search_head_patterns"]
