"""Pins for the oracle's automatic prefix caching ("What is paged attention
in vLLM...", Trade-offs and edge cases, fourth point: full blocks are hashed,
the least recently used are evicted).

Each check holds whatever the bookkeeping: a repeated prompt finds the
blocks its first request filled; a change in an early block hides every
later block (keys are chained); at least one prompt token is always left
to compute; evictable blocks leave in least-recently-used order, and only
when no free block is left; attention through cached blocks equals
attention through freshly written ones.  Planted mistakes must each trip a
check.
"""

import numpy as np
import pytest

from oracle import attention as oatt
from oracle import cache_ops as oc
from oracle.allocator import (BlockAllocator, InvalidArgument, OutOfBlocks, block_key,
                              fnv1a64)

BS = 4


def test_fnv1a64_published_vectors():
    # Test vectors of the FNV-1a 64-bit function as published by its authors.
    assert fnv1a64(b"") == 0xCBF29CE484222325
    assert fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert fnv1a64(b"foobar") == 0x85944171F73967E8


def _run(a, sid, tokens):
    """create + match + reserve the rest; returns the tokens found cached."""
    a.seq_create(sid)
    hit = a.match_prefix(sid, tokens)
    a.seq_reserve([sid], [len(tokens) - hit])
    return hit


def check_repeat_hits(cls):
    a = cls(32, BS)
    a.enable_prefix_cache()
    p = list(range(100, 122))  # 22 tokens: 5 full blocks + 2
    assert _run(a, 0, p) == 0
    first = a.seq_block_table(0)
    a.seq_free(0)
    assert a.num_cached() == 5 and sorted(a.cached_list()) == sorted(first[:5])
    assert _run(a, 1, p + [7, 8, 9]) == 20
    assert a.seq_block_table(1)[:5] == first[:5] and a.num_cached() == 0
    assert a.seq_num_tokens(1) == 25


def check_one_token_left(cls):
    a = cls(32, BS)
    a.enable_prefix_cache()
    p = list(range(16))  # exactly 4 full blocks
    _run(a, 0, p)
    a.seq_free(0)
    assert _run(a, 1, p) == 12  # 3 blocks; the last block is computed again


def check_chained_keys(cls):
    a = cls(32, BS)
    a.enable_prefix_cache()
    p = list(range(50, 70))
    _run(a, 0, p)
    a.seq_free(0)
    q = [999] + p[1:]  # block 0 differs, blocks 1-4 are equal
    assert _run(a, 1, q + [1]) == 0
    assert block_key(0, p[:4]) != block_key(0, q[:4])
    assert block_key(block_key(0, p[:4]), p[4:8]) != block_key(block_key(0, q[:4]), p[4:8])
    # Cached [X, Y] and [Z, W]: a prompt [X, W] may take X but not W, whose
    # cached block followed another prefix.
    X, Y, Z, Wt = [1] * 4, [2] * 4, [3] * 4, [4] * 4
    _run(a, 2, X + Y + [0])
    _run(a, 3, Z + Wt + [0])
    a.seq_free(2)
    a.seq_free(3)
    assert _run(a, 4, X + Wt + [0]) == 4


def check_live_sharing(cls):
    a = cls(32, BS)
    a.enable_prefix_cache()
    p = list(range(10))  # 2 full blocks + 2 in the tail
    _run(a, 0, p)
    assert _run(a, 1, p + [3]) == 8  # A is still running: its full blocks are shared
    t0, t1 = a.seq_block_table(0), a.seq_block_table(1)
    assert t0[:2] == t1[:2] and [a.refcount(b) for b in t0[:2]] == [2, 2]
    assert t0[2] != t1[2]
    slots, pairs = a.seq_reserve([0, 1], [1, 1])
    assert pairs == []  # full blocks are never written, so never copied


def check_free_first_then_lru(cls):
    a = cls(12, BS)
    a.enable_prefix_cache()
    for sid, base in ((0, 100), (1, 200), (2, 300)):
        _run(a, sid, list(range(base, base + 8)) + [0])  # 2 full blocks each
    order = []
    for sid in (1, 0, 2):  # released in this order
        blocks = a.seq_block_table(sid)[:2]
        a.seq_free(sid)
        order += list(reversed(blocks))
    assert a.cached_list() == order and a.num_free() == 12 - 6
    a.seq_create(9)
    a.seq_reserve([9], [6 * BS])  # takes the 6 free blocks: nothing evicted
    assert a.cached_list() == order
    a.seq_reserve([9], [3 * BS])  # 3 more: the 3 least recently released go
    assert a.cached_list() == order[3:]
    a.seq_create(10)
    assert a.match_prefix(10, list(range(200, 208)) + [0]) == 0  # sequence 1's blocks: evicted
    a.seq_create(11)
    assert a.match_prefix(11, list(range(100, 108)) + [0]) == 4  # sequence 0: block 1 evicted
    a.seq_create(12)
    assert a.match_prefix(12, list(range(300, 308)) + [0]) == 8  # sequence 2's: still cached


def check_rollback_keeps_cache(cls):
    a = cls(6, BS)
    a.enable_prefix_cache()
    _run(a, 0, list(range(12)) + [0])
    a.seq_free(0)
    snap = (a.free_list(), a.cached_list(), [a.refcount(b) for b in range(6)])
    a.seq_create(1)
    with pytest.raises(OutOfBlocks):
        a.seq_reserve([1], [7 * BS])
    assert (a.free_list(), a.cached_list(), [a.refcount(b) for b in range(6)]) == snap
    assert a.match_prefix(1, list(range(12)) + [5]) == 12


def check_failed_reserve_keeps_evicted_keys(cls):
    """A reserve that evicts a cached block, refills it (registering a new
    key on it) and then runs out of blocks must give the block its old key
    back: afterwards the old prompt still hits and the new one does not."""
    a = cls(1, 2)
    a.enable_prefix_cache()
    a.seq_create(0)
    assert a.match_prefix(0, [1, 2, 3]) == 0
    a.seq_reserve([0], [2])  # block 0 full: cached under the key of [1, 2]
    a.seq_free(0)
    assert a.cached_list() == [0] and a.block_key(0) == block_key(0, [1, 2])
    a.seq_create(1)
    assert a.match_prefix(1, [5, 6, 7]) == 0
    with pytest.raises(OutOfBlocks):
        a.seq_reserve([1], [3])  # evicts block 0, fills it with [5, 6], needs a 2nd
    assert a.cached_list() == [0] and a.num_free() == 0
    assert a.block_key(0) == block_key(0, [1, 2])
    a.seq_free(1)
    a.seq_create(2)
    assert a.match_prefix(2, [5, 6, 7]) == 0
    a.seq_free(2)
    a.seq_create(3)
    assert a.match_prefix(3, [1, 2, 3]) == 2 and a.seq_block_table(3) == [0]


def check_errors(cls):
    a = cls(8, BS)
    a.seq_create(0)
    with pytest.raises(InvalidArgument):
        a.match_prefix(0, [1, 2, 3, 4, 5])  # cache off
    a.enable_prefix_cache()
    a.seq_reserve([0], [2])
    with pytest.raises(InvalidArgument):
        a.match_prefix(0, [1, 2, 3, 4, 5])  # not empty


PREFIX_PINS = [check_repeat_hits, check_one_token_left, check_chained_keys, check_live_sharing,
               check_free_first_then_lru, check_rollback_keeps_cache,
               check_failed_reserve_keeps_evicted_keys, check_errors]


@pytest.mark.parametrize("pin", PREFIX_PINS, ids=lambda f: f.__name__)
def test_prefix_pin(pin):
    pin(BlockAllocator)


def test_attention_through_cached_blocks_equals_fresh_blocks():
    """Request B reuses A's cached prompt blocks; its decode equals the decode
    of the same tokens written into fresh blocks (bit-exact)."""
    rng = np.random.default_rng(4)
    HKV, D, nb = 2, 16, 40
    prompt = list(rng.integers(0, 1000, 21))
    rows = {t: (rng.standard_normal((HKV, D)).astype(np.float32),
                rng.standard_normal((HKV, D)).astype(np.float32)) for t in set(prompt) | {7}}

    def write(a, kc, vc, sid, tokens, start):
        slots, _ = a.seq_reserve([sid], [len(tokens) - start])
        k = np.stack([rows[t][0] for t in tokens[start:]])
        v = np.stack([rows[t][1] for t in tokens[start:]])
        oc.cache_append(kc, vc, k, v, slots, BS)

    q = rng.standard_normal((1, 2 * HKV, D)).astype(np.float32)
    outs = []
    for cached in (True, False):
        a = BlockAllocator(nb, BS, free_order=rng.permutation(nb))
        kc = np.full((nb, HKV, BS, D), np.nan, np.float32)
        vc = kc.copy()
        if cached:
            a.enable_prefix_cache()
            a.seq_create(0)
            a.match_prefix(0, prompt)
            write(a, kc, vc, 0, prompt, 0)
            a.seq_free(0)
        b = prompt + [7]
        a.seq_create(1)
        hit = a.match_prefix(1, b) if cached else 0
        assert hit == (20 if cached else 0)
        write(a, kc, vc, 1, b, hit)
        t, lens = a.block_tables([1], 8)
        outs.append(oatt.paged_decode(q, kc, vc, np.array(t), np.array(lens), BS, 0.25, "f32"))
    assert np.array_equal(outs[0], outs[1])


# ------------------------------------------------------------ planted mistakes
class _Unchained(BlockAllocator):
    """Keys and the hit check use the block's own tokens only (no parent)."""

    def match_prefix(self, seq_id, tokens):
        toks = [int(t) for t in tokens]
        bs = self.block_size
        keys = []
        for i in range(len(toks) // bs):
            blk_toks = tuple(toks[i * bs:(i + 1) * bs])
            keys.append((block_key(0, blk_toks), 0, blk_toks))
        self._keys[seq_id] = keys
        hits = 0
        for key, parent, blk_toks in keys[:(len(toks) - 1) // bs if toks else 0]:
            blk = self._block_of.get(key)
            if blk is None or self._key_of[blk] != (key, parent, blk_toks):
                break
            if self._rc[blk] == 0:
                self._lru.remove(blk)
            self._rc[blk] += 1
            self._table[seq_id].append(blk)
            hits += 1
        self._ntok[seq_id] = hits * bs
        return hits * bs


class _EvictNewest(BlockAllocator):
    def _pop(self):
        if not self._free and self._lru:
            self._lru.insert(0, self._lru.pop())
        return super()._pop()


class _NoTokenLeft(BlockAllocator):
    """May take every full block of the prompt."""

    def match_prefix(self, seq_id, tokens):
        return super().match_prefix(seq_id, list(tokens) + [0])


class _EvictFirst(BlockAllocator):
    """Evicts a cached block even while free blocks remain."""

    def _pop(self):
        if self._lru:
            saved, self._free = self._free, []
            try:
                return super()._pop()
            finally:
                self._free = saved
        return super()._pop()


class _NoCaching(BlockAllocator):
    """Released cached blocks go straight back to the free stack."""

    def _release(self, blk):
        self._rc[blk] -= 1
        if self._rc[blk] == 0:
            self._free.append(blk)


def _fails(pin, cls):
    try:
        pin(cls)
    except (AssertionError, OutOfBlocks, InvalidArgument, KeyError, ValueError,
            pytest.fail.Exception):
        return True
    return False


@pytest.mark.parametrize("cls", [_Unchained, _EvictNewest, _NoTokenLeft, _EvictFirst, _NoCaching],
                         ids=lambda c: c.__name__)
def test_planted_prefix_mistake_is_caught(cls):
    assert any(_fails(pin, cls) for pin in PREFIX_PINS), cls.__name__
