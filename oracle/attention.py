"""Oracle single-query (decode) attention, float64.

Paging changes where the cache lives, not the attention arithmetic
["PagedAttention — AI Glossary", Example: the gain comes with no change to
the attention mathematics; "What is paged attention in vLLM...", Common
mistakes, first item].  So the oracle is the textbook definition

    s_p   = scale * <q, k_p>           for every context position p < L
    w_p   = exp(s_p - max_p s_p)
    out   = sum_p w_p v_p / sum_p w_p

with K/V rows found through the block table: position p lives in logical
block p // bs at offset p % bs, and the table maps the logical block to a
physical block ["Paged Attention" glossary, body; "What is paged attention
in vLLM...", Step 3].

Readings adopted where the pages are silent:
* grouped-query attention maps query head h to KV head h // G with
  G = num_q_heads / num_kv_heads (consecutive grouping);
* a sequence with zero context gives an all-zero output row;
* stored values are widened to float64 exactly before any arithmetic
  (bf16 is held as uint16 bit patterns).

Three independent formulations are provided so they can pin one another:
``paged_decode`` (gather through the table, numpy), ``contiguous_decode``
(contiguous logical rows, scipy's softmax) and ``brute_force_decode``
(scalar Python with math.exp / math.fsum).
"""

from __future__ import annotations

import math

import numpy as np
from scipy.special import softmax


def widen(x, dtype: str):
    """Stored values -> float64, exactly.  ``dtype`` is 'f32', 'bf16' or 'f16'
    (IEEE binary16, held as uint16 bit patterns like bf16)."""
    x = np.asarray(x)
    if dtype == "f16":
        if x.dtype != np.uint16:
            raise TypeError("f16 values are passed as uint16 bit patterns")
        return x.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        if x.dtype != np.uint16:
            raise TypeError("bf16 values are passed as uint16 bit patterns")
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "f32":
        if x.dtype != np.float32:
            raise TypeError("f32 values are passed as float32")
        return x.astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def paged_decode(q, k_cache, v_cache, block_tables, context_lens, block_size,
                 scale, dtype):
    """Decode attention reading K/V through per-sequence block tables.

    q            [B, H_q, D]                     stored dtype
    k/v_cache    [num_blocks, H_kv, bs, D]       stored dtype
    block_tables [B, max_blocks] int (entries past the length are ignored)
    context_lens [B] int
    returns      [B, H_q, D] float64
    """
    qf = widen(q, dtype)
    B, H_q, D = qf.shape
    H_kv = k_cache.shape[1]
    G = H_q // H_kv
    tables = np.asarray(block_tables, dtype=np.int64)
    lens = np.asarray(context_lens, dtype=np.int64)
    out = np.zeros((B, H_q, D), dtype=np.float64)
    for b in range(B):
        L = int(lens[b])
        if L == 0:
            continue
        pos = np.arange(L)
        phys = tables[b, pos // block_size]
        off = pos % block_size
        for kvh in range(H_kv):
            K = widen(k_cache[phys, kvh, off, :], dtype)  # [L, D]
            V = widen(v_cache[phys, kvh, off, :], dtype)
            for g in range(G):
                h = kvh * G + g
                s = scale * (K @ qf[b, h])
                w = np.exp(s - s.max())
                out[b, h] = (w @ V) / w.sum()
    return out


def contiguous_decode(q, k_seqs, v_seqs, scale, dtype):
    """Same attention over contiguous per-sequence caches (no table).

    ``k_seqs[b]``/``v_seqs[b]`` are ``[L_b, H_kv, D]`` in logical order: the
    cache a contiguous (slab) layout would hold ["Paged Attention" glossary,
    definition: the table lets attention read the context as if it were
    continuous].
    """
    qf = widen(q, dtype)
    B, H_q, D = qf.shape
    out = np.zeros((B, H_q, D), dtype=np.float64)
    for b in range(B):
        K = widen(k_seqs[b], dtype)
        V = widen(v_seqs[b], dtype)
        if K.shape[0] == 0:
            continue
        H_kv = K.shape[1]
        G = H_q // H_kv
        for h in range(H_q):
            kvh = h // G
            p = softmax(scale * (K[:, kvh, :] @ qf[b, h]))
            out[b, h] = p @ V[:, kvh, :]
    return out


def brute_force_decode(q, k_cache, v_cache, block_tables, context_lens,
                       block_size, scale, dtype):
    """Scalar loops, ``math.exp`` and ``math.fsum``: tiny inputs only."""
    qf = widen(q, dtype).tolist()
    Kf = widen(k_cache, dtype)
    Vf = widen(v_cache, dtype)
    B, H_q, D = len(qf), len(qf[0]), len(qf[0][0])
    H_kv = Kf.shape[1]
    G = H_q // H_kv
    out = [[[0.0] * D for _ in range(H_q)] for _ in range(B)]
    for b in range(B):
        L = int(context_lens[b])
        for h in range(H_q):
            kvh = h // G
            rows = []
            for p in range(L):
                blk = int(block_tables[b][p // block_size])
                rows.append((Kf[blk, kvh, p % block_size].tolist(),
                             Vf[blk, kvh, p % block_size].tolist()))
            if not rows:
                continue
            logits = [scale * math.fsum(a * c for a, c in zip(qf[b][h], k))
                      for k, _ in rows]
            top = max(logits)
            w = [math.exp(s - top) for s in logits]
            den = math.fsum(w)
            for d in range(D):
                out[b][h][d] = math.fsum(wi * v[d] for wi, (_, v) in zip(w, rows)) / den
    return np.array(out, dtype=np.float64)
