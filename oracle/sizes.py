"""KV-cache sizing formulas.  TEST INFRASTRUCTURE ONLY.

* Per-token KV bytes: two tensors (K and V) per layer, each holding one vector of
  ``head_dim`` elements per KV head -- "LLM inference optimization: KV cache &
  PagedAttention" (carlstack.gravito.dev), section 1.2 (KV cache size estimate).
  That page writes the head count as ``n_heads``; its worked example (Llama 3 70B)
  uses 8, the number of KV heads, so the factor is the KV-head count.
* Per-block bytes: the same product times ``block_size`` tokens -- "vLLM explained"
  (jackchen890311.github.io), section on how block size is decided, block-byte formula.
* Number of blocks: memory available for KV divided by the block bytes, rounded
  down -- same section, closing paragraph.
* Internal fragmentation: the unused tail of each sequence's last block -- "LLM
  inference optimization" section 二.2 (fragmentation taxonomy) and "vLLM explained",
  block-size trade-off table (small blocks waste less inside a block).
"""


def kv_bytes_per_token(num_layers, num_kv_heads, head_dim, elem_bytes):
    """Bytes of K plus V for one token across all layers."""
    return 2 * num_layers * num_kv_heads * head_dim * elem_bytes


def block_bytes(block_size, num_layers, num_kv_heads, head_dim, elem_bytes):
    """Bytes of one physical block: ``block_size`` tokens of K and V in every layer."""
    return block_size * kv_bytes_per_token(num_layers, num_kv_heads, head_dim, elem_bytes)


def num_blocks_for_memory(kv_memory_bytes, bytes_per_block):
    """How many whole blocks fit into ``kv_memory_bytes``."""
    return kv_memory_bytes // bytes_per_block


def blocks_needed(context_len, block_size):
    """Blocks a sequence of ``context_len`` tokens occupies (last block may be partial)."""
    return -(-context_len // block_size)


def internal_waste_fraction(context_lens, block_size):
    """Fraction of allocated token slots that hold no token (exact rational as float)."""
    allocated = sum(blocks_needed(L, block_size) * block_size for L in context_lens)
    used = sum(context_lens)
    return 0.0 if allocated == 0 else (allocated - used) / allocated
