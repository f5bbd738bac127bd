"""The pages' memory arithmetic, written out (integers and exact fractions).

These are the figures the pages print for the contiguous ("slab") layout
that paging replaces and for the block layout, so the tests can pin both the
formulas and the allocator against the printed numbers.
"""

from __future__ import annotations

from fractions import Fraction


def kv_bytes_per_token(num_layers, num_kv_heads, head_dim, bytes_per_value):
    """K and V for every layer and KV head: 2 * layers * heads * dim * bytes.

    "What is paged attention in vLLM...", Step 1 prices one token of a
    32-layer, 8-KV-head, head-size-128 model (2-byte values implied).
    """
    return 2 * num_layers * num_kv_heads * head_dim * bytes_per_value


def blocks_for(tokens, block_size):
    """Blocks a sequence of ``tokens`` holds under lazy allocation.

    A block is taken only when the last one is full, so the count is the
    ceiling of tokens / block_size ("What is paged attention in vLLM...",
    Step 4; "PagedAttention — AI Glossary", Example).
    """
    if tokens < 0 or block_size < 1:
        raise ValueError("tokens >= 0 and block_size >= 1 required")
    return -(-tokens // block_size)


def tail_waste(tokens, block_size):
    """Idle slots at the end of the last block: always below one block."""
    return blocks_for(tokens, block_size) * block_size - tokens


def slab_utilisation(lengths, max_len):
    """Share of slots holding tokens when each request reserves max_len."""
    lengths = [int(x) for x in lengths]
    return Fraction(sum(lengths), len(lengths) * max_len)


def paged_utilisation(lengths, block_size):
    """Share of allocated block slots holding tokens."""
    lengths = [int(x) for x in lengths]
    slots = sum(blocks_for(x, block_size) * block_size for x in lengths)
    return Fraction(sum(lengths), slots)


def slab_capacity(cache_bytes, max_len, bytes_per_token):
    """Requests that fit when each reserves a max_len slab."""
    return int(cache_bytes // (max_len * bytes_per_token))


def paged_capacity(cache_bytes, lengths, block_size, bytes_per_token):
    """Requests that fit when each holds the batch's mean allocated slots.

    "What is paged attention in vLLM...", Worked example: capacity under
    blocks at the example batch's average size.
    """
    lengths = [int(x) for x in lengths]
    slots = sum(blocks_for(x, block_size) * block_size for x in lengths)
    mean_slots = Fraction(slots, len(lengths))
    return int(Fraction(cache_bytes) // (mean_slots * bytes_per_token))
