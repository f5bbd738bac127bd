"""Oracle cache writes: slot-mapped append and whole-block copy.

Both are exact bit copies, so they work on any numpy dtype (float32 values,
or bf16 values held as uint16 bit patterns).

Pool layout (a reading; the pages only say that a block holds the keys and
values of a fixed number of tokens): separate K and V pools, each shaped
``[num_blocks, num_kv_heads, block_size, head_dim]``.
"""

from __future__ import annotations

import numpy as np


def cache_append(k_cache, v_cache, k, v, slot_mapping, block_size):
    """Write token t's K/V rows into the slot ``slot_mapping[t]``.

    At every decode step the new token's keys and values go into the last
    block of its sequence; during prefill the prompt tokens fill fresh blocks
    the same way ["What is paged attention in vLLM...", Step 4;
    "Paged Attention" glossary, body].  A slot is ``block * block_size +
    offset``; a negative slot means "no write" (padding).

    ``k``/``v`` are ``[T, num_kv_heads, head_dim]``; the pools are modified
    in place.  Non-negative slots must be distinct (two writes to one slot
    in one call have no defined order).
    """
    slots = np.asarray(slot_mapping, dtype=np.int64).reshape(-1)
    live = slots[slots >= 0]
    if len(np.unique(live)) != len(live):
        raise ValueError("duplicate slot in one append")
    n_slots = k_cache.shape[0] * block_size
    if len(live) and live.max() >= n_slots:
        raise ValueError("slot beyond the pool")
    for t, s in enumerate(slots.tolist()):
        if s < 0:
            continue
        blk, off = divmod(s, block_size)
        k_cache[blk, :, off, :] = k[t]
        v_cache[blk, :, off, :] = v[t]


def copy_blocks(k_cache, v_cache, src_dst_pairs):
    """Copy whole blocks ``src -> dst`` in both pools.

    Copy-on-write duplicates only the block being written when a shared
    sequence diverges ["PagedAttention — AI Glossary", How it works, item 5;
    "What is paged attention in vLLM...", Trade-offs and edge cases, third
    point].  Every slot of the block is copied, filled or not.
    """
    pairs = np.asarray(src_dst_pairs, dtype=np.int64).reshape(-1, 2)
    for s, d in pairs.tolist():
        k_cache[d] = k_cache[s]
        v_cache[d] = v_cache[s]


def swap_blocks(src_k, src_v, dst_k, dst_v, src_dst_pairs):
    """Copy whole blocks from one pool pair to another: ``dst[d] = src[s]``.

    A preempted sequence's blocks move to CPU memory and back ["What is
    paged attention in vLLM...", Follow-up questions, "What happens when the
    GPU runs out of free blocks?": blocks are swapped to CPU memory or
    dropped and recomputed; "Paged Attention" glossary, Common questions,
    "What happens when the GPU runs out of KV blocks?"].  The two pools have the same
    block geometry and may differ in block count.
    """
    pairs = np.asarray(src_dst_pairs, dtype=np.int64).reshape(-1, 2)
    for s, d in pairs.tolist():
        dst_k[d] = src_k[s]
        dst_v[d] = src_v[s]
