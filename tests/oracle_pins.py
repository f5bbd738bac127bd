"""Pin checks for the oracle, written so they also run against deliberately
broken copies of it (tests/test_oracle_mutations.py): each check takes the
implementation under test as an argument and raises AssertionError on a
mismatch.  Expected values come from the pages (tests/golden), closed forms,
scipy, or brute force - never from the oracle itself.
"""

from __future__ import annotations

import math

import numpy as np


def _f32(x):
    return np.asarray(x, dtype=np.float32)


# ---------------------------------------------------------------- allocator
def check_seven_token_prompt(alloc_cls):
    """Step 3 of the clozo.ai page: 7 tokens, 4 per block -> physical 7 and 1."""
    order = [7, 1] + [x for x in range(16) if x not in (7, 1)]
    a = alloc_cls(16, 4, order)
    a.seq_create(0)
    slots, pairs = a.seq_reserve([0], [7])
    assert a.seq_block_table(0) == [7, 1]
    assert list(slots) == [28, 29, 30, 31, 4, 5, 6]
    assert list(pairs) == []
    free_before = a.num_free()
    slots, _ = a.seq_reserve([0], [1])       # the waiting last slot
    assert list(slots) == [7] and a.num_free() == free_before
    slots, _ = a.seq_reserve([0], [1])       # now the block is full: take order[2]
    assert a.seq_block_table(0) == [7, 1, order[2]]
    assert list(slots) == [order[2] * 4]


def check_worked_batch(alloc_cls, figures):
    wb = figures["worked_batch"]
    bs = wb["block_size"]
    a = alloc_cls(4096, bs, None)
    for i, L in enumerate(wb["lengths"]):
        a.seq_create(i)
        a.seq_reserve([i], [L])
    blocks = sum(len(a.seq_block_table(i)) for i in range(len(wb["lengths"])))
    tokens = sum(a.seq_num_tokens(i) for i in range(len(wb["lengths"])))
    assert tokens == wb["tokens"]
    assert blocks * bs == wb["paged_slots"]
    assert round(100 * tokens / (blocks * bs), 1) == wb["paged_used_percent"]
    assert a.num_free() == 4096 - blocks


def check_600_and_700(alloc_cls, figures):
    ex = figures["slab_vs_blocks_600"]
    a = alloc_cls(1024, ex["block_size"], None)
    a.seq_create(0)
    a.seq_reserve([0], [ex["average_tokens"]])
    assert len(a.seq_block_table(0)) == ex["blocks"]
    r = figures["request_700"]
    a.seq_create(1)
    a.seq_reserve([1], [r["tokens"]])
    nb = len(a.seq_block_table(1))
    assert nb == r["blocks"] and nb * r["block_size"] == r["slots"]
    assert nb * r["block_size"] - a.seq_num_tokens(1) == r["idle_slots"]


def check_free_lifo_reuse(alloc_cls):
    """Freed blocks are handed out again at once, logical block 0 first."""
    a = alloc_cls(32, 4, list(range(31, -1, -1)))
    a.seq_create(0)
    a.seq_reserve([0], [10])
    t0 = a.seq_block_table(0)
    a.seq_free(0)
    a.seq_create(1)
    a.seq_reserve([1], [10])
    assert a.seq_block_table(1) == t0


def check_fork_cow_trace(alloc_cls):
    """Hand-derived trace of fork + copy-on-write (block size 4).

    seq 0 gets 6 tokens -> blocks [0, 1] (block 1 half full).  Forking twice
    gives counts 3/3.  Seq 1 then writes one token into the shared, partly
    filled block 1: it is copied to the next free block (2); seq 2 does the
    same (-> 3); seq 0, by then the only holder of block 1, writes in place.
    """
    a = alloc_cls(8, 4, None)
    a.seq_create(0)
    slots, pairs = a.seq_reserve([0], [6])
    assert list(slots) == [0, 1, 2, 3, 4, 5] and list(pairs) == []
    a.seq_fork(0, 1)
    a.seq_fork(0, 2)
    assert [a.refcount(b) for b in (0, 1)] == [3, 3]
    slots, pairs = a.seq_reserve([1, 2, 0], [1, 1, 1])
    assert [tuple(p) for p in pairs] == [(1, 2), (1, 3)]
    assert list(slots) == [2 * 4 + 2, 3 * 4 + 2, 1 * 4 + 2]
    assert a.seq_block_table(1) == [0, 2]
    assert a.seq_block_table(2) == [0, 3]
    assert a.seq_block_table(0) == [0, 1]
    assert [a.refcount(b) for b in range(4)] == [3, 1, 1, 1]
    # Seq 1 fills its private copy of block 1, then takes a fresh block.
    slots, pairs = a.seq_reserve([1], [3])
    assert list(pairs) == [] and list(slots) == [11, 16, 17]
    # Seq 0 fills block 1; a fork then shares a FULL tail, and the fork's
    # next token takes a fresh block instead of copying.
    slots, _ = a.seq_reserve([0], [1])
    assert list(slots) == [7]
    a.seq_fork(0, 3)
    assert [a.refcount(b) for b in (0, 1)] == [4, 2]
    slots, pairs = a.seq_reserve([3], [1])
    assert list(pairs) == [] and list(slots) == [5 * 4]
    # Freeing seq 1 returns its private blocks; its logical block 1 comes out first.
    a.seq_free(1)
    assert a.free_list()[:3] == [2, 4, 6]
    assert a.refcount(0) == 3


def check_out_of_blocks_rollback(alloc_cls, out_of_blocks_exc):
    a = alloc_cls(4, 4, None)
    a.seq_create(0)
    a.seq_create(1)
    a.seq_reserve([0], [5])
    before = (a.free_list(), [a.refcount(b) for b in range(4)],
              a.seq_block_table(0), a.seq_block_table(1))
    try:
        a.seq_reserve([0, 1], [3, 9])
    except out_of_blocks_exc:
        pass
    else:
        raise AssertionError("expected out-of-blocks")
    after = (a.free_list(), [a.refcount(b) for b in range(4)],
             a.seq_block_table(0), a.seq_block_table(1))
    assert before == after
    a.seq_free(0)
    a.seq_reserve([1], [9])  # the freed blocks are usable at once
    assert len(a.seq_block_table(1)) == 3


# ------------------------------------------------------------------ decode
def check_two_token_closed_form(decode_fn):
    """q=(2,0), keys (0,0),(1,0), scale 1/2 -> logits (0,1) -> logistic weights."""
    q = _f32([[[2.0, 0.0]]])
    kc = _f32(np.zeros((2, 1, 1, 2)))
    vc = _f32(np.zeros((2, 1, 1, 2)))
    kc[1, 0, 0] = [1.0, 0.0]
    vc[0, 0, 0] = [1.0, 0.0]
    vc[1, 0, 0] = [0.0, 1.0]
    out = decode_fn(q, kc, vc, np.array([[0, 1]]), np.array([2]), 1, 0.5, "f32")
    e = math.e
    np.testing.assert_allclose(out[0, 0], [1 / (1 + e), e / (1 + e)], rtol=0, atol=1e-15)


def check_gqa_grouping(decode_fn):
    """KV head j holds constant values c_j: query head h must return c_{h//G}."""
    H_q, H_kv, D, bs = 6, 3, 4, 2
    rng = np.random.default_rng(0)
    q = rng.standard_normal((1, H_q, D)).astype(np.float32)
    kc = rng.standard_normal((3, H_kv, bs, D)).astype(np.float32)
    vc = np.zeros((3, H_kv, bs, D), dtype=np.float32)
    for j in range(H_kv):
        vc[:, j] = float(j + 1)
    out = decode_fn(q, kc, vc, np.array([[2, 0, 1]]), np.array([5]), bs, 0.3, "f32")
    for h in range(H_q):
        np.testing.assert_allclose(out[0, h], np.full(D, float(h // 2 + 1)), rtol=0, atol=1e-12)


def check_single_token_is_v(decode_fn):
    rng = np.random.default_rng(1)
    q = rng.standard_normal((2, 2, 8)).astype(np.float32)
    kc = rng.standard_normal((5, 1, 4, 8)).astype(np.float32)
    vc = rng.standard_normal((5, 1, 4, 8)).astype(np.float32)
    out = decode_fn(q, kc, vc, np.array([[3], [1]]), np.array([1, 1]), 4, 0.7, "f32")
    for h in range(2):
        assert np.array_equal(out[0, h], vc[3, 0, 0].astype(np.float64))
        assert np.array_equal(out[1, h], vc[1, 0, 0].astype(np.float64))


def check_zero_query_mean(decode_fn):
    rng = np.random.default_rng(2)
    L, bs = 11, 4
    q = np.zeros((1, 1, 8), dtype=np.float32)
    kc = rng.standard_normal((4, 1, bs, 8)).astype(np.float32)
    vc = rng.standard_normal((4, 1, bs, 8)).astype(np.float32)
    table = np.array([[2, 0, 3]])
    out = decode_fn(q, kc, vc, table, np.array([L]), bs, 1.0, "f32")
    rows = [vc[table[0, p // bs], 0, p % bs].astype(np.float64) for p in range(L)]
    np.testing.assert_allclose(out[0, 0], np.mean(rows, axis=0), rtol=0, atol=1e-14)


def check_scaled_two_block_vs_scipy(decode_fn):
    """Random case across blocks vs scipy.special.softmax on hand-gathered rows."""
    from scipy.special import softmax
    rng = np.random.default_rng(3)
    bs, D, L = 4, 16, 10
    q = rng.standard_normal((1, 1, D)).astype(np.float32)
    kc = rng.standard_normal((6, 1, bs, D)).astype(np.float32)
    vc = rng.standard_normal((6, 1, bs, D)).astype(np.float32)
    table = [5, 0, 2]
    Kl = np.stack([kc[table[p // bs], 0, p % bs] for p in range(L)]).astype(np.float64)
    Vl = np.stack([vc[table[p // bs], 0, p % bs] for p in range(L)]).astype(np.float64)
    expect = softmax(0.25 * (Kl @ q[0, 0].astype(np.float64))) @ Vl
    out = decode_fn(q, kc, vc, np.array([table]), np.array([L]), bs, 0.25, "f32")
    np.testing.assert_allclose(out[0, 0], expect, rtol=0, atol=1e-13)


# ------------------------------------------------------------------- cache ops
def check_append_places_rows(append_fn):
    kc = np.zeros((3, 2, 4, 2), dtype=np.float32)
    vc = np.zeros_like(kc)
    k = np.arange(3 * 2 * 2, dtype=np.float32).reshape(3, 2, 2) + 1
    v = -k
    append_fn(kc, vc, k, v, [9, -1, 2], 4)   # slot 9 = block 2 offset 1
    assert np.array_equal(kc[2, :, 1, :], k[0]) and np.array_equal(vc[2, :, 1, :], v[0])
    assert np.array_equal(kc[0, :, 2, :], k[2]) and np.array_equal(vc[0, :, 2, :], v[2])
    assert np.count_nonzero(kc) == 8  # two tokens x 2 heads x 2 dims, nothing else


def check_copy_whole_block(copy_fn):
    kc = np.arange(4 * 2 * 3 * 2, dtype=np.float32).reshape(4, 2, 3, 2)
    vc = -kc
    before = kc.copy()
    copy_fn(kc, vc, [(1, 3), (0, 2)])
    assert np.array_equal(kc[3], before[1]) and np.array_equal(kc[2], before[0])
    assert np.array_equal(vc[3], -before[1]) and np.array_equal(kc[:2], before[:2])
