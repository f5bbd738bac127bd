"""Oracle multi-query (prefill / chunked prefill) attention, float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

During prefill a prompt's blocks are allocated and filled, and decoding then
continues from that state ["Paged Attention" glossary, body; "What is paged
attention in vLLM...", Step 3: the 7-token prompt fills logical blocks 0 and
1].  The attention arithmetic over those tokens is the ordinary causal one;
paging only changes where the rows are found ["PagedAttention — AI
Glossary", Example].  So the oracle is the textbook definition, with K/V rows
gathered through the block table exactly as in the decode oracle:

    sequence b holds L_b tokens in the cache; its n_b query tokens are the
    last n_b positions, the i-th at position p_i = L_b - n_b + i, and

    s_t   = scale * <q_i, k_t>        for t <= p_i      (causal)
    out_i = sum_t exp(s_t - max s) v_t / sum_t exp(s_t - max s)

Readings adopted where the pages are silent:
* the query tokens' own keys and values are already in the cache (appended
  first), so a query attends to itself;
* n_b = 1 for every sequence is exactly decode;
* grouped-query attention maps query head h to KV head h // G;
* query rows of all sequences are packed: sequence b's rows are
  q[query_start[b] : query_start[b + 1]], and n_b <= L_b.

Two formulations are given so they can pin each other: ``paged_prefill``
(gather through the table, one softmax per query row) and
``dense_causal_prefill`` (contiguous logical rows, one masked score matrix
per sequence and head, scipy's softmax).  ``brute_force_prefill`` is scalar
Python for tiny inputs.
"""

from __future__ import annotations

import math

import numpy as np
from scipy.special import softmax

from .attention import widen


def _check_starts(query_start, context_lens):
    qs = np.asarray(query_start, dtype=np.int64)
    lens = np.asarray(context_lens, dtype=np.int64)
    n = np.diff(qs)
    if qs[0] != 0 or (n < 0).any() or (n > lens).any():
        raise ValueError("query_start must start at 0, increase, and n_b <= L_b")
    return qs, lens


def paged_prefill(q, k_cache, v_cache, block_tables, context_lens, query_start,
                  block_size, scale, dtype):
    """Causal multi-query attention reading K/V through block tables.

    q            [T, H_q, D] stored dtype, T = query_start[-1]
    k/v_cache    [num_blocks, H_kv, bs, D] stored dtype
    block_tables [B, max_blocks] int
    context_lens [B] int (the cache length, query tokens included)
    query_start  [B + 1] int, packed query rows per sequence
    returns      [T, H_q, D] float64
    """
    qf = widen(q, dtype)
    T, H_q, D = qf.shape
    H_kv = k_cache.shape[1]
    G = H_q // H_kv
    qs, lens = _check_starts(query_start, context_lens)
    tables = np.asarray(block_tables, dtype=np.int64)
    out = np.zeros((T, H_q, D), dtype=np.float64)
    for b in range(len(lens)):
        L, n = int(lens[b]), int(qs[b + 1] - qs[b])
        if n == 0:
            continue
        pos = np.arange(L)
        phys = tables[b, pos // block_size]
        off = pos % block_size
        for kvh in range(H_kv):
            K = widen(k_cache[phys, kvh, off, :], dtype)  # [L, D] in logical order
            V = widen(v_cache[phys, kvh, off, :], dtype)
            for i in range(n):
                p = L - n + i  # position of query token i
                for g in range(G):
                    h = kvh * G + g
                    s = scale * (K[: p + 1] @ qf[qs[b] + i, h])
                    w = np.exp(s - s.max())
                    out[qs[b] + i, h] = (w @ V[: p + 1]) / w.sum()
    return out


def dense_causal_prefill(q, k_seqs, v_seqs, query_start, scale, dtype):
    """The same attention as one masked score matrix per (sequence, head).

    ``k_seqs[b]``/``v_seqs[b]`` are ``[L_b, H_kv, D]`` in logical order (the
    contiguous cache the table stands for).  Scores of keys after a query's
    own position are set to -inf before scipy's softmax.
    """
    qf = widen(q, dtype)
    T, H_q, D = qf.shape
    qs = np.asarray(query_start, dtype=np.int64)
    out = np.zeros((T, H_q, D), dtype=np.float64)
    for b in range(len(k_seqs)):
        K = widen(k_seqs[b], dtype)
        V = widen(v_seqs[b], dtype)
        L, n = K.shape[0], int(qs[b + 1] - qs[b])
        if n == 0:
            continue
        H_kv = K.shape[1]
        G = H_q // H_kv
        qpos = np.arange(L - n, L)[:, None]
        mask = np.arange(L)[None, :] > qpos  # [n, L]: key after the query
        for h in range(H_q):
            S = scale * (qf[qs[b]:qs[b + 1], h] @ K[:, h // G, :].T)
            S[mask] = -np.inf
            out[qs[b]:qs[b + 1], h] = softmax(S, axis=1) @ V[:, h // G, :]
    return out


def brute_force_prefill(q, k_cache, v_cache, block_tables, context_lens, query_start,
                        block_size, scale, dtype):
    """Scalar loops with ``math.exp`` and ``math.fsum``: tiny inputs only."""
    qf = widen(q, dtype).tolist()
    Kf = widen(k_cache, dtype)
    Vf = widen(v_cache, dtype)
    T, H_q, D = len(qf), len(qf[0]), len(qf[0][0])
    G = H_q // Kf.shape[1]
    out = [[[0.0] * D for _ in range(H_q)] for _ in range(T)]
    for b in range(len(context_lens)):
        L = int(context_lens[b])
        n = int(query_start[b + 1]) - int(query_start[b])
        for i in range(n):
            row = int(query_start[b]) + i
            for h in range(H_q):
                rows = []
                for t in range(L - n + i + 1):
                    blk = int(block_tables[b][t // block_size])
                    rows.append((Kf[blk, h // G, t % block_size].tolist(),
                                 Vf[blk, h // G, t % block_size].tolist()))
                logits = [scale * math.fsum(a * c for a, c in zip(qf[row][h], k)) for k, _ in rows]
                top = max(logits)
                w = [math.exp(s - top) for s in logits]
                den = math.fsum(w)
                for d in range(D):
                    out[row][h][d] = math.fsum(wi * v[d] for wi, (_, v) in zip(w, rows)) / den
    return np.array(out, dtype=np.float64)


def prefill_flops(context_lens, query_start, num_q_heads, head_dim):
    """Algorithmic multiply-add work of one call: every (query row, key) pair
    the causal mask keeps costs 2*D flops for q.k and 2*D for p.v."""
    qs = np.asarray(query_start, dtype=np.int64)
    total = 0
    for b, L in enumerate(np.asarray(context_lens, dtype=np.int64)):
        n = int(qs[b + 1] - qs[b])
        # keys seen by the n query rows: (L - n + 1) + ... + L
        total += n * (L - n) + n * (n + 1) // 2
    return int(total) * num_q_heads * 4 * head_dim
