"""The oracle reproduces every figure the pages print (tests/golden)."""

from fractions import Fraction

import oracle_pins as pins
from oracle import accounting as acc
from oracle.allocator import BlockAllocator, OutOfBlocks


def test_seven_token_prompt():
    pins.check_seven_token_prompt(BlockAllocator)


def test_worked_batch_allocator(page_figures):
    pins.check_worked_batch(BlockAllocator, page_figures)


def test_600_and_700_token_requests(page_figures):
    pins.check_600_and_700(BlockAllocator, page_figures)


def test_free_lifo_reuse():
    pins.check_free_lifo_reuse(BlockAllocator)


def test_fork_cow_trace():
    pins.check_fork_cow_trace(BlockAllocator)


def test_out_of_blocks_rollback():
    pins.check_out_of_blocks_rollback(BlockAllocator, OutOfBlocks)


def test_slab_example_600(page_figures):
    ex = page_figures["slab_vs_blocks_600"]
    assert acc.blocks_for(ex["average_tokens"], ex["block_size"]) == ex["blocks"]
    used = acc.slab_utilisation([ex["average_tokens"]], ex["reserved_tokens"])
    assert round(100 * float(used)) == ex["used_percent_about"]
    assert round(100 * float(1 - used)) == ex["idle_percent_about"]


def test_llama3_bytes(page_figures):
    f = page_figures["llama3_8b_cache_bytes"]
    bpt = acc.kv_bytes_per_token(f["layers"], f["kv_heads"], f["head_size"], 2)
    assert bpt == f["bytes_per_token"] == 128 * 1024
    assert bpt * f["max_positions"] == f["bytes_per_full_reservation"] == 2 ** 30


def test_request_700(page_figures):
    r = page_figures["request_700"]
    used = acc.slab_utilisation([r["tokens"]], 8192)
    assert round(100 * float(used), 1) == r["slab_used_percent"]
    assert round(100 * float(1 - used), 1) == r["slab_wasted_percent"]
    assert acc.blocks_for(r["tokens"], r["block_size"]) == r["blocks"]
    assert acc.tail_waste(r["tokens"], r["block_size"]) == r["idle_slots"]
    held = r["blocks"] * r["block_size"]
    assert held == r["slots"]
    assert round(100 * r["idle_slots"] / held, 2) == r["idle_percent"]


def test_worked_batch_accounting(page_figures):
    wb = page_figures["worked_batch"]
    L = wb["lengths"]
    assert sum(L) == wb["tokens"]
    assert len(L) * wb["slab_max_len"] == wb["slab_slots"]
    assert round(100 * float(acc.slab_utilisation(L, wb["slab_max_len"])), 1) == wb["slab_used_percent"]
    pu = acc.paged_utilisation(L, wb["block_size"])
    assert pu == Fraction(wb["tokens"], wb["paged_slots"])
    assert round(100 * float(pu), 1) == wb["paged_used_percent"]
    # Lazy allocation matters: 128 tokens are exactly 8 blocks.  Taking a
    # block ahead of need would give 10,656 slots, not the printed 10,640.
    assert acc.blocks_for(128, 16) == 8
    eager = sum((x // 16 + 1) * 16 for x in L)
    assert eager == 10656 != wb["paged_slots"]


def test_capacity_64gb(page_figures):
    wb = page_figures["worked_batch"]
    bpt = acc.kv_bytes_per_token(32, 8, 128, 2)
    slab = acc.slab_capacity(wb["cache_bytes"], wb["slab_max_len"], bpt)
    paged = acc.paged_capacity(wb["cache_bytes"], wb["lengths"], wb["block_size"], bpt)
    assert slab == wb["slab_requests"]
    assert paged == wb["paged_requests_about"]
    assert round(paged / slab, 1) == wb["ratio"]


def test_tail_waste_below_one_block():
    import random
    rnd = random.Random(7)
    for _ in range(2000):
        bs = rnd.choice([1, 2, 4, 8, 16, 32, 128])
        L = rnd.randrange(0, 5000)
        w = acc.tail_waste(L, bs)
        assert 0 <= w <= bs - 1
        a = BlockAllocator(-(-L // bs) + 1, bs)
        a.seq_create(0)
        a.seq_reserve([0], [L])
        assert len(a.seq_block_table(0)) * bs - L == w
