"""Slot-mapped K/V writes and whole-block copies, as bit copies.  TEST INFRASTRUCTURE ONLY.

Pool layout (one layer): ``[num_blocks][num_kv_heads][block_size][head_dim]`` raw
bits, K and V in separate arrays; a multi-layer pool stacks
``[num_layers][2 (K, V)][num_blocks][num_kv_heads][block_size][head_dim]``.

* ``reshape_and_cache``: a new token's K/V rows go to the physical slot that the
  block manager assigned to it, ``slot = block * block_size + offset``; slot -1
  means "no write".  Blocks are allocated on demand and filled token by token --
  "vLLM explained" (jackchen890311.github.io), PagedAttention section, item 4;
  "LLM inference optimization" (carlstack.gravito.dev), block-mapping figure
  (logical block 2 mapped to a physical block allocated on demand).
* ``copy_blocks``: copy-on-write copies a whole shared block when a branch first
  writes a different token into it -- carlstack page, section 三.2 and Fig. 1.
  The whole block is copied, in every layer, K and V, in the order the pairs are
  given.
"""

import numpy as np


def reshape_and_cache(k_pool, v_pool, k_new, v_new, slots, block_size):
    """Write rows ``k_new[i], v_new[i]`` (``[T][H_kv][d]`` raw bits) into one layer's pools.

    ``k_pool, v_pool``: ``[N][H_kv][bs][d]`` raw-bit arrays, modified in place.
    """
    for i, slot in enumerate(np.asarray(slots).tolist()):
        if slot < 0:
            continue
        block, offset = divmod(slot, block_size)
        k_pool[block, :, offset, :] = k_new[i]
        v_pool[block, :, offset, :] = v_new[i]


def copy_blocks(pool, pairs):
    """``pool[..., dst, ...] <- pool[..., src, ...]`` for every (src, dst), in order.

    ``pool``: ``[num_layers][2][N][H_kv][bs][d]`` raw bits, modified in place.
    """
    for src, dst in np.asarray(pairs).reshape(-1, 2).tolist():
        pool[:, :, dst] = pool[:, :, src]
