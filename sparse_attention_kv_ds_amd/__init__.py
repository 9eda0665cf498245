"""MI355X-native lightning indexer (DeepSeek V4 sparse attention): score every
query token against the causally visible compressed KV rows and keep the
top-k rows per token, on hand-written HIP kernels for gfx950.

The compute path lives in the C-ABI library ``libds_indexer.so`` (built from
``csrc/``); ``sparse_attention_kv_ds_amd.indexer`` is its thin Python binding.
``sparse_attention_kv_ds_amd.synth`` holds the seeded input generators.
"""

__all__ = ["indexer", "synth"]
