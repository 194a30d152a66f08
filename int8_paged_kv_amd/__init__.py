"""int8 paged KV cache for AMD MI355X (gfx950).

Operations behind the C ABI of libq8kv.so (include/q8kv.h):

* ``q8_cache_write``: symmetric per-token int8 quantize + pack of new K/V
  vectors into the paged cache (the "reshape_and_cache_q8.comp" page).
* ``q8_paged_decode``: single-query decode attention over that cache (the
  "paged_attn_q8.comp" page), optionally over per-sequence visible-position
  lists (the selective decode of the "attention.rs" page).
* ``q8_paged_decode_noalloc``: the same decode with the library's own
  scratch array in place of a workspace, for callers that cannot allocate.
* ``q8_decode_step``: both in one launch for the usual decode step (each
  sequence's new token appended at its last position, then attended).
* ``q8_paged_decode_rows``: multi-row causal decode (several query rows per
  sequence at its last positions, each over its causal prefix).
* ``q8_f32_cache_write`` / ``q8_f32_paged_decode`` and ``q8_bf16_cache_write`` /
  ``q8_bf16_paged_decode``: the same write and decode over f32 and bfloat16 paged
  caches, the baselines the int8 cache is measured against.
* ``q8_rope_table``, ``q8_norm_rope``, ``q8_norm_rope_cache_write``: per-head
  RMSNorm + partial rotary embedding of q rows, and fused ahead of the K
  quantizer in the cache write (the q/k norm-and-rope step of "attention.rs");
  ``q8_norm_rope_qk_cache_write`` does the q rows and the K/V write in one launch,
  ``q8_norm_rope_decode_step`` the whole step (norm + rotary, append, decode).
* ``q8_index_select``: block scores to visible-position lists (the top
  kblk blocks plus the trailing partial block), the input of the visible-list
  decode.

The binding loads the library lazily, so ``int8_paged_kv_amd.workloads`` can
be imported on a machine without the library or a GPU.
"""

__all__ = ["q8_cache_write", "q8_paged_decode", "q8_paged_decode_noalloc", "q8_decode_step", "q8_paged_decode_rows",
           "q8_paged_decode_workspace_bytes", "q8_f32_cache_write", "q8_f32_paged_decode",
           "q8_f32_paged_decode_workspace_bytes", "q8_bf16_cache_write", "q8_bf16_paged_decode",
           "q8_bf16_paged_decode_workspace_bytes", "q8_rope_table", "q8_norm_rope", "q8_norm_rope_cache_write",
           "q8_norm_rope_qk_cache_write", "q8_norm_rope_decode_step", "q8_index_select",
           "load_library", "load_debug_library", "use_library", "bounds_flags", "Q8Error", "PAD_SLOT"]


def __getattr__(name):
    if name in __all__:
        from . import _binding
        return getattr(_binding, name)
    raise AttributeError(name)
