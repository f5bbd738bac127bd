"""Pins for the oracle's preemption paths: a host (CPU memory) block pool,
swap-out and swap-in of whole sequences, and drop-and-recompute.

The pages state the mechanism only ("Paged Attention" glossary, Common
questions, "What happens when the GPU runs out of KV blocks?"; "What is
paged attention in vLLM...", Follow-up questions, "What happens when the GPU
runs out of free blocks?"): a preempted request's blocks are moved to CPU
memory, or dropped and recomputed in one prefill pass.  What must hold
whatever the bookkeeping: the attention output after a round trip is the
output before it, bit for bit (it reads the same values through another
table); a sequence's sharers keep their blocks; block counts add up; a call
that cannot complete changes nothing.  Each check below is also run against
copies of the oracle with a planted mistake, which it must catch.
"""

import numpy as np
import pytest

from oracle import attention as oatt
from oracle import cache_ops as oc
from oracle.allocator import BlockAllocator, InvalidArgument, OutOfBlocks

BS, NB, NH, HKV, D = 8, 40, 30, 2, 16


def _state(a):
    return (a.free_list(), [a.refcount(i) for i in range(a.num_blocks)],
            {s: a.seq_block_table(s) for s in a.seq_ids()},
            {s: a.seq_num_tokens(s) for s in a.seq_ids()},
            a.host_free_list(), {s: a.seq_is_swapped(s) for s in a.seq_ids()})


def _filled(cls, lengths=(37, 16, 70), seed=0, nh=NH):
    """Allocator (with a host pool) holding the given sequences, device and
    host pools, and the K rows of every sequence in logical order."""
    rng = np.random.default_rng(seed)
    a = cls(NB, BS, free_order=rng.permutation(NB))
    a.add_host_pool(nh, free_order=rng.permutation(nh))
    kc = np.full((NB, HKV, BS, D), np.nan, np.float32)
    vc = np.full((NB, HKV, BS, D), np.nan, np.float32)
    hk = np.full((nh, HKV, BS, D), np.nan, np.float32)
    hv = np.full((nh, HKV, BS, D), np.nan, np.float32)
    for s, L in enumerate(lengths):
        a.seq_create(s)
        slots, _ = a.seq_reserve([s], [L])
        oc.cache_append(kc, vc, rng.standard_normal((L, HKV, D)).astype(np.float32),
                        rng.standard_normal((L, HKV, D)).astype(np.float32), slots, BS)
    return a, kc, vc, hk, hv


def _decode(a, kc, vc, seqs, q):
    rows, lens = a.block_tables(seqs, 16)
    return oatt.paged_decode(q, kc, vc, np.array(rows), np.array(lens), BS, 0.25, "f32")


def _q(n, seed=9):
    return np.random.default_rng(seed).standard_normal((n, 2 * HKV, D)).astype(np.float32)


def check_round_trip_is_bit_exact(cls):
    """Swap sequence 1 out, let another sequence take (and overwrite) the
    released device blocks, swap it back in: decode output unchanged."""
    a, kc, vc, hk, hv = _filled(cls)
    q = _q(3)
    before = _decode(a, kc, vc, [0, 1, 2], q)
    oc.swap_blocks(kc, vc, hk, hv, a.swap_out(1))
    a.seq_create(7)
    slots, _ = a.seq_reserve([7], [16])  # reuses the released blocks
    oc.cache_append(kc, vc, np.full((16, HKV, D), 7.0, np.float32),
                    np.full((16, HKV, D), -7.0, np.float32), slots, BS)
    assert np.array_equal(_decode(a, kc, vc, [0, 2], q[[0, 2]]), before[[0, 2]])
    oc.swap_blocks(hk, hv, kc, vc, a.swap_in(1))
    after = _decode(a, kc, vc, [0, 1, 2], q)
    assert np.array_equal(after, before)


def check_counts(cls):
    a, kc, vc, hk, hv = _filled(cls)
    n1 = len(a.seq_block_table(1))
    free0, host0 = a.num_free(), a.num_free_host()
    pairs = a.swap_out(1)
    assert len(pairs) == n1 and a.num_free() == free0 + n1 and a.num_free_host() == host0 - n1
    assert sorted(h for _, h in pairs) == sorted(a.seq_block_table(1))
    a.swap_in(1)
    assert a.num_free() == free0 and a.num_free_host() == host0
    live = [s for s in a.seq_ids() if not a.seq_is_swapped(s)]
    assert sum(a.refcount(i) for i in range(NB)) == sum(len(a.seq_block_table(s)) for s in live)
    assert a.num_free() + sum(a.refcount(i) > 0 for i in range(NB)) == NB


def check_shared_blocks_stay(cls):
    """A forked child swapped out: the parent keeps every block (count back
    to 1), its bytes untouched by later allocations; the child's copy comes
    back in private blocks."""
    a, kc, vc, hk, hv = _filled(cls, lengths=(37,))
    a.seq_fork(0, 1)
    parent = a.seq_block_table(0)
    q = _q(1)
    before = _decode(a, kc, vc, [0], q)
    oc.swap_blocks(kc, vc, hk, hv, a.swap_out(1))
    assert a.seq_block_table(0) == parent and all(a.refcount(b) == 1 for b in parent)
    assert not set(parent) & set(a.free_list())
    a.seq_create(5)
    slots, _ = a.seq_reserve([5], [a.num_free() * BS])  # take every free block
    oc.cache_append(kc, vc, np.zeros((len(slots), HKV, D), np.float32),
                    np.zeros((len(slots), HKV, D), np.float32), slots, BS)
    assert np.array_equal(_decode(a, kc, vc, [0], q), before)
    a.seq_free(5)
    oc.swap_blocks(hk, hv, kc, vc, a.swap_in(1))
    assert not set(a.seq_block_table(1)) & set(parent)
    assert np.array_equal(_decode(a, kc, vc, [1], q), before)


def check_all_or_nothing(cls):
    a, *_ = _filled(cls, nh=4)  # sequence 2 needs 9 host blocks
    s0 = _state(a)
    with pytest.raises(OutOfBlocks):
        a.swap_out(2)
    assert _state(a) == s0
    a2, *_ = _filled(cls, lengths=(70, 30))
    a2.swap_out(0)
    a2.seq_create(3)
    a2.seq_reserve([3], [(a2.num_free() - 4) * BS])  # leave 4 free blocks, 9 needed
    s1 = _state(a2)
    with pytest.raises(OutOfBlocks):
        a2.swap_in(0)
    assert _state(a2) == s1


def check_lifo_orders(cls):
    """Host blocks come off the host stack in its order; swap-in takes the
    device blocks on top of the device stack; a freed swapped sequence puts
    its logical block 0 on top of the host stack."""
    a, *_ = _filled(cls)
    top_host = a.host_free_list()
    pairs = a.swap_out(2)
    assert [h for _, h in pairs] == top_host[:len(pairs)]
    top_dev = a.free_list()
    back = a.swap_in(2)
    assert [d for _, d in back] == top_dev[:len(back)]
    pairs = a.swap_out(0)
    host0 = [h for _, h in pairs]
    a.seq_free(0)
    assert a.host_free_list()[:len(host0)] == host0


def check_errors(cls):
    a, *_ = _filled(cls)
    a.swap_out(1)
    for bad in (lambda: a.swap_out(1), lambda: a.seq_reserve([1], [1]), lambda: a.seq_fork(1, 9),
                lambda: a.block_tables([1], 16), lambda: a.swap_in(0),
                lambda: a.add_host_pool(4)):
        with pytest.raises(InvalidArgument):
            bad()
    b = cls(4, 4)
    b.seq_create(0)
    with pytest.raises(InvalidArgument):
        b.swap_out(0)  # no host pool


SWAP_PINS = [check_round_trip_is_bit_exact, check_counts, check_shared_blocks_stay,
             check_all_or_nothing, check_lifo_orders, check_errors]


@pytest.mark.parametrize("pin", SWAP_PINS, ids=lambda f: f.__name__)
def test_swap_pin(pin):
    pin(BlockAllocator)


def test_drop_and_recompute_is_bit_exact():
    """The other preemption path: free the sequence, create it again, reserve
    its tokens and write the same K/V rows (the prefill pass): decode output
    is unchanged, whatever blocks it now holds."""
    rng = np.random.default_rng(3)
    a = BlockAllocator(NB, BS, free_order=rng.permutation(NB))
    kc = np.full((NB, HKV, BS, D), np.nan, np.float32)
    vc = kc.copy()
    rows = {}
    for s, L in enumerate((37, 50)):
        a.seq_create(s)
        slots, _ = a.seq_reserve([s], [L])
        rows[s] = (rng.standard_normal((L, HKV, D)).astype(np.float32),
                   rng.standard_normal((L, HKV, D)).astype(np.float32))
        oc.cache_append(kc, vc, *rows[s], slots, BS)
    q = _q(2)
    before = _decode(a, kc, vc, [0, 1], q)
    a.seq_free(0)
    a.seq_create(6)
    a.seq_reserve([6], [20])  # someone else takes the blocks first
    a.seq_create(0)
    slots, _ = a.seq_reserve([0], [37])
    oc.cache_append(kc, vc, *rows[0], slots, BS)
    assert np.array_equal(_decode(a, kc, vc, [0, 1], q), before)


# ------------------------------------------------------------ planted mistakes
class _SwapFreesShared(BlockAllocator):
    """Swap-out releases every device block, shared or not."""

    def swap_out(self, seq_id):
        table = list(self._table[seq_id])
        pairs = super().swap_out(seq_id)
        for blk in reversed(table):
            if self._rc[blk] > 0:
                self._rc[blk] = 0
                self._free.append(blk)
        return pairs


class _SwapInNoCount(BlockAllocator):
    """Swap-in forgets the counts of the new device blocks."""

    def swap_in(self, seq_id):
        pairs = super().swap_in(seq_id)
        for _, d in pairs:
            self._rc[d] = 0
        return pairs


class _HostFifo(BlockAllocator):
    """Host blocks taken from the bottom of the host stack."""

    def swap_out(self, seq_id):
        if self._host_free is None:
            return super().swap_out(seq_id)
        self._host_free.reverse()
        try:
            return super().swap_out(seq_id)
        finally:
            self._host_free.reverse()


class _SwapInPartial(BlockAllocator):
    """Swap-in takes device blocks until it runs out, then raises."""

    def swap_in(self, seq_id):
        need = len(self._table[seq_id])
        if need > len(self._free):
            while self._free:
                self._rc[self._free.pop()] = 1
            raise OutOfBlocks("no free block")
        return super().swap_in(seq_id)


class _SwapOutKeepsRefs(BlockAllocator):
    """Swap-out never releases the device blocks."""

    def swap_out(self, seq_id):
        table = list(self._table[seq_id])
        rc = [self._rc[b] for b in table]
        free = list(self._free)
        pairs = super().swap_out(seq_id)
        self._free = free
        for b, r in zip(table, rc):
            self._rc[b] = r
        return pairs


def _fails(pin, cls):
    try:
        pin(cls)
    except (AssertionError, OutOfBlocks, InvalidArgument, KeyError, IndexError,
            pytest.fail.Exception):
        return True
    return False


@pytest.mark.parametrize("cls", [_SwapFreesShared, _SwapInNoCount, _HostFifo, _SwapInPartial,
                                 _SwapOutKeepsRefs], ids=lambda c: c.__name__)
def test_planted_swap_mistake_is_caught(cls):
    assert any(_fails(pin, cls) for pin in SWAP_PINS), cls.__name__
