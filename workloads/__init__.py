"""Seeded synthetic inputs for the paged-KV decode path.

This module only draws inputs.  It holds none of the method's arithmetic (no
slot, table, copy or attention computation) and imports neither the oracle nor
the HIP binding, so both sides can be fed from it.

Every workload is described by
* shapes (heads, head size, block size, value type) and the softmax scale;
* a pool size and ``free_order``: the seeded permutation in which a fresh
  allocator hands blocks out (this is how "blocks scattered in the pool" is
  produced: consecutive logical blocks land on random physical blocks);
* ``q`` and a bank of K/V rows drawn i.i.d. N(0, 1) in float32 (bf16
  workloads round them to bf16 by round-to-nearest-even on the bit pattern
  and store the bits as uint16);
* ``script``: the allocator calls that build the cache - ``("create", sid)``,
  ``("fork", parent, child)`` and ``("reserve", sids, n_new, rows)`` where
  ``rows`` indexes the K/V bank for the new tokens, sequence-major in call
  order, i.e. exactly the rows to append at the returned slots;
* ``seq_ids`` (decode batch order) and ``logical_rows[b]``: bank indices of
  sequence b's tokens in logical order (what a contiguous cache would hold).

Draw order within one workload: lengths, free_order, q, K, V (K and V
sequence-major, logical order).  ``with_values=False`` skips q/K/V (for
allocator-only use); everything drawn before them is unchanged.  Pools start filled with NaN bit patterns so
that a read of an unwritten slot shows up.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

POISON_BITS = {"f32": np.uint32(0x7FC00000), "bf16": np.uint16(0x7FC0), "f16": np.uint16(0x7E00)}
STORAGE = {"f32": np.float32, "bf16": np.uint16, "f16": np.uint16}
BYTES = {"f32": 4, "bf16": 2, "f16": 2}


def round_to_bf16_bits(x):
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = bits + np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def round_to_f16_bits(x):
    """float32 -> IEEE binary16 bit patterns (uint16), round to nearest even."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def _normal(rng, shape, dtype, draw=True):
    if not draw:
        return None
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == "bf16":
        return round_to_bf16_bits(x)
    return round_to_f16_bits(x) if dtype == "f16" else x


@dataclass
class Workload:
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str
    scale: float
    num_blocks: int
    free_order: np.ndarray
    q: np.ndarray
    k_rows: np.ndarray
    v_rows: np.ndarray
    script: list
    seq_ids: list
    logical_rows: list
    notes: dict = field(default_factory=dict)

    @property
    def batch(self):
        return len(self.seq_ids)

    @property
    def context_lens(self):
        return np.array([len(r) for r in self.logical_rows], dtype=np.int64)

    def empty_pool(self):
        """One NaN-poisoned pool ``[num_blocks, H_kv, bs, D]`` (K or V)."""
        shape = (self.num_blocks, self.num_kv_heads, self.block_size, self.head_dim)
        bits = np.full(shape, POISON_BITS[self.dtype])
        return bits.view(STORAGE[self.dtype]) if self.dtype == "f32" else bits

    def kv_bytes(self):
        """Bytes of K and V a decode pass must read (valid tokens only)."""
        return int(self.context_lens.sum()) * 2 * self.num_kv_heads * self.head_dim * BYTES[self.dtype]


def _sequential_script(lengths, first_row=0):
    """Create every sequence, then fill each one in batch order, one call each."""
    script = [("create", b) for b in range(len(lengths))]
    logical, start = [], first_row
    for b, L in enumerate(lengths):
        rows = np.arange(start, start + L, dtype=np.int64)
        script.append(("reserve", [b], [int(L)], rows))
        logical.append(rows)
        start += L
    return script, logical


def _round_robin_script(lengths, block_size):
    """Fill all sequences in lock step, one block's worth of tokens per round.

    Sequences that grow together interleave their blocks in the pool.
    """
    lengths = [int(x) for x in lengths]
    offs = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    script = [("create", b) for b in range(len(lengths))]
    done = [0] * len(lengths)
    while True:
        sids, ns, rows = [], [], []
        for b, L in enumerate(lengths):
            n = min(block_size, L - done[b])
            if n > 0:
                sids.append(b)
                ns.append(n)
                rows.append(np.arange(offs[b] + done[b], offs[b] + done[b] + n, dtype=np.int64))
                done[b] += n
        if not sids:
            break
        script.append(("reserve", sids, ns, np.concatenate(rows)))
    logical = [np.arange(offs[b], offs[b + 1], dtype=np.int64) for b in range(len(lengths))]
    return script, logical


def tiny_ref(seed=1, with_values=True):
    """4 sequences of 7/16/33/100 tokens, 4 Q / 2 KV heads, head 64, bs 4, fp32."""
    lengths = [7, 16, 33, 100]
    rng = np.random.default_rng(seed)
    nb, bs, hq, hkv, d = 64, 4, 4, 2, 64
    free_order = rng.permutation(nb).astype(np.int32)
    q = _normal(rng, (len(lengths), hq, d), "f32", with_values)
    tot = sum(lengths)
    k = _normal(rng, (tot, hkv, d), "f32", with_values)
    v = _normal(rng, (tot, hkv, d), "f32", with_values)
    script, logical = _sequential_script(lengths)
    return Workload("tiny_ref", seed, hq, hkv, d, bs, "f32", 1.0 / 8.0, nb, free_order,
                    q, k, v, script, list(range(len(lengths))), logical)


LLAMA3_8B_BATCH = [128, 700, 1500, 300, 2900, 50, 4100, 900]


def llama3_8b_decode(seed=2, lengths=None, num_blocks=4096, block_size=16, with_values=True):
    """One Llama-3-8B attention layer at decode: 32 Q / 8 KV heads, head 128.

    Default lengths are the eight-request batch of the worked example in
    "What is paged attention in vLLM..." (10,578 tokens).  ``new_k``/``new_v``
    in ``notes`` hold one extra token per sequence for a decode step.
    """
    lengths = list(LLAMA3_8B_BATCH if lengths is None else lengths)
    rng = np.random.default_rng(seed)
    hq, hkv, d = 32, 8, 128
    free_order = rng.permutation(num_blocks).astype(np.int32)
    q = _normal(rng, (len(lengths), hq, d), "bf16", with_values)
    tot = sum(lengths)
    k = _normal(rng, (tot, hkv, d), "bf16", with_values)
    v = _normal(rng, (tot, hkv, d), "bf16", with_values)
    new_k = _normal(rng, (len(lengths), hkv, d), "bf16", with_values)
    new_v = _normal(rng, (len(lengths), hkv, d), "bf16", with_values)
    script, logical = _sequential_script(lengths)
    return Workload("llama3_8b_decode", seed, hq, hkv, d, block_size, "bf16",
                    1.0 / math.sqrt(d), num_blocks, free_order, q, k, v, script,
                    list(range(len(lengths))), logical,
                    notes={"new_k": new_k, "new_v": new_v})


def serving_batch(seed=3, batch=256, with_values=True):
    """256 sequences, log-normal lengths (mean 600, sigma 1, capped at 8192),
    interleaved in a pool of ceil(1.1 * total / 16) blocks, then one appended
    token per sequence before the decode.
    """
    rng = np.random.default_rng(seed)
    bs, hq, hkv, d = 16, 32, 8, 128
    raw = rng.lognormal(mean=math.log(600.0) - 0.5, sigma=1.0, size=batch)
    lengths = np.clip(np.rint(raw), 1, 8192).astype(np.int64).tolist()
    total = sum(lengths)
    nb = -(-(11 * total) // (10 * bs))
    assert nb >= sum(-(-(L + 1) // bs) for L in lengths)
    free_order = rng.permutation(nb).astype(np.int32)
    q = _normal(rng, (batch, hq, d), "bf16", with_values)
    k = _normal(rng, (total + batch, hkv, d), "bf16", with_values)
    v = _normal(rng, (total + batch, hkv, d), "bf16", with_values)
    script, logical = _round_robin_script(lengths, bs)
    new_rows = np.arange(total, total + batch, dtype=np.int64)
    script.append(("reserve", list(range(batch)), [1] * batch, new_rows))
    logical = [np.concatenate([logical[b], new_rows[b:b + 1]]) for b in range(batch)]
    return Workload("serving_batch", seed, hq, hkv, d, bs, "bf16", 1.0 / math.sqrt(d),
                    nb, free_order, q, k, v, script, list(range(batch)), logical,
                    notes={"prefill_lengths": lengths})


BLOCK_SIZE_SWEEP = (8, 16, 32, 128)


def block_size_sweep(block_size, seed=4, batch=64, max_len=8192, with_values=True):
    """64 sequences with lengths uniform on [1, 8192]; same lengths and values
    for every block size, pool ceil(1.1 * blocks needed), shuffled per size.
    """
    if block_size not in BLOCK_SIZE_SWEEP:
        raise ValueError("block size outside the sweep")
    rng = np.random.default_rng(seed)
    hq, hkv, d = 32, 8, 128
    lengths = rng.integers(1, max_len + 1, size=batch).tolist()
    needed = sum(-(-L // block_size) for L in lengths)
    nb = -(-(11 * needed) // 10)
    free_order = np.random.default_rng(seed * 1000 + block_size).permutation(nb).astype(np.int32)
    q = _normal(rng, (batch, hq, d), "bf16", with_values)
    tot = sum(lengths)
    k = _normal(rng, (tot, hkv, d), "bf16", with_values)
    v = _normal(rng, (tot, hkv, d), "bf16", with_values)
    script, logical = _sequential_script(lengths)
    return Workload(f"block_size_sweep_bs{block_size}", seed, hq, hkv, d, block_size, "bf16",
                    1.0 / math.sqrt(d), nb, free_order, q, k, v, script,
                    list(range(batch)), logical)


def prefix_sharing(seed=5, batch=128, prefix_len=2056, max_suffix=512, with_values=True):
    """128 sequences forked from one prefix, each with its own suffix.

    Sequence 0 is filled with the prefix and forked 127 times, so every
    prefix block is shared by all 128 sequences.  One call then reserves
    each sequence's suffix (uniform 0..512 tokens) plus one decode token.
    With the default prefix of 2,056 tokens the prefix ends half way into a
    16-token block, so that first call must copy the shared tail block for
    every sequence but the last; with a prefix of 2,048 it ends on a block
    boundary and nothing is copied.
    """
    rng = np.random.default_rng(seed)
    bs, hq, hkv, d = 16, 32, 8, 128
    suffix = rng.integers(0, max_suffix + 1, size=batch).tolist()
    grow = [s + 1 for s in suffix]
    held = prefix_len // bs + sum(-(-(prefix_len + g) // bs) - (prefix_len // bs) for g in grow)
    nb = -(-(11 * held) // 10)
    free_order = rng.permutation(nb).astype(np.int32)
    q = _normal(rng, (batch, hq, d), "bf16", with_values)
    tot = prefix_len + sum(grow)
    k = _normal(rng, (tot, hkv, d), "bf16", with_values)
    v = _normal(rng, (tot, hkv, d), "bf16", with_values)
    prefix_rows = np.arange(prefix_len, dtype=np.int64)
    script = [("create", 0), ("reserve", [0], [prefix_len], prefix_rows)]
    script += [("fork", 0, c) for c in range(1, batch)]
    offs = np.concatenate([[prefix_len], prefix_len + np.cumsum(grow)]).astype(np.int64)
    suffix_rows = np.arange(prefix_len, tot, dtype=np.int64)
    script.append(("reserve", list(range(batch)), grow, suffix_rows))
    logical = [np.concatenate([prefix_rows, np.arange(offs[b], offs[b + 1], dtype=np.int64)])
               for b in range(batch)]
    return Workload(f"prefix_sharing_p{prefix_len}", seed, hq, hkv, d, bs, "bf16",
                    1.0 / math.sqrt(d), nb, free_order, q, k, v, script,
                    list(range(batch)), logical,
                    notes={"prefix_len": prefix_len, "suffix": suffix, "held_blocks": held})


CONFIGS = {
    "tiny_ref": tiny_ref,
    "llama3_8b_decode": llama3_8b_decode,
    "serving_batch": serving_batch,
    "block_size_sweep": block_size_sweep,
    "prefix_sharing": prefix_sharing,
}
