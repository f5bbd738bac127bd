"""Preemption on the GPU: block moves between a device pool and a pinned
host pool (pa_swap_blocks), the C allocator's swap-out / swap-in, and the
drop-and-recompute path, against the oracle (needs a gfx950 GPU).

Block moves are bit copies and must be bit-exact.  A preempted sequence
that comes back (swapped in to other device blocks, or recomputed into
other blocks) must give decode output bit-identical to before: the decode
kernel's arithmetic depends on the logical layout only, never on physical
block ids.
"""

import numpy as np
import pytest

import parity_log
import workloads as W
from oracle import cache_ops as ocops
from oracle_driver import OracleCache

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import paged_kv_cache_338_amd as pa
    pa.load_library()
    yield


def _gd():
    import gpu_driver
    return gpu_driver


def _pinned(a, dtype):
    return _gd().to_torch(a, dtype, "cpu").pin_memory()


@pytest.mark.parametrize("dtype,shape", [("bf16", (40, 8, 16, 128)), ("f32", (12, 2, 4, 64)),
                                         ("f16", (12, 2, 8, 64))])
@pytest.mark.parametrize("pairs_on", ["device", "pinned"])
def test_swap_blocks_bit_exact_both_directions(dtype, shape, pairs_on):
    import torch
    import paged_kv_cache_338_amd as pa
    gd = _gd()
    rng = np.random.default_rng(21)
    nh = 9
    k, v = W._normal(rng, shape, dtype), W._normal(rng, shape, dtype)
    poison = W.POISON_BITS[dtype]
    hshape = (nh,) + shape[1:]
    hk = np.full(hshape, poison, np.uint32 if dtype == "f32" else np.uint16)
    if dtype == "f32":
        hk = hk.view(np.float32)
    hv = hk.copy()
    out_pairs = np.array([[3, 7], [0, 5], [9, 0], [11, 8]], np.int32)
    dk, dv = gd.to_torch(k, dtype, "cuda:0"), gd.to_torch(v, dtype, "cuda:0")
    tk, tv = _pinned(hk, dtype), _pinned(hv, dtype)

    def pairs_t(p):
        t = torch.from_numpy(p)
        return t.cuda() if pairs_on == "device" else t.pin_memory()

    pa.pa_swap_blocks(pairs_t(out_pairs), dk, dv, tk, tv)
    torch.cuda.synchronize()
    ocops.swap_blocks(k, v, hk, hv, out_pairs)
    assert np.array_equal(gd.to_numpy(tk, dtype).view(np.uint8), hk.view(np.uint8))
    assert np.array_equal(gd.to_numpy(tv, dtype).view(np.uint8), hv.view(np.uint8))
    # Back in, to other blocks of a second (poisoned) device pool.
    k2 = np.full(shape, poison, hk.dtype)
    v2 = k2.copy()
    in_pairs = np.array([[7, 1], [5, 2], [0, 3], [8, 4]], np.int32)
    dk2, dv2 = gd.to_torch(k2, dtype, "cuda:0"), gd.to_torch(v2, dtype, "cuda:0")
    pa.pa_swap_blocks(pairs_t(in_pairs), tk, tv, dk2, dv2)
    torch.cuda.synchronize()
    ocops.swap_blocks(hk, hv, k2, v2, in_pairs)
    assert np.array_equal(gd.to_numpy(dk2, dtype).view(np.uint8), k2.view(np.uint8))
    assert np.array_equal(gd.to_numpy(dv2, dtype).view(np.uint8), v2.view(np.uint8))
    assert np.array_equal(k2[1:5], k[[3, 0, 9, 11]])


def test_swap_blocks_skips_out_of_pool_ids():
    import torch
    import paged_kv_cache_338_amd as pa
    gd = _gd()
    shape = (6, 2, 8, 64)
    k = W._normal(np.random.default_rng(2), shape, "bf16")
    h = np.full((4,) + shape[1:], W.POISON_BITS["bf16"], np.uint16)
    tk, tv = _pinned(h, "bf16"), _pinned(h, "bf16")
    dk = gd.to_torch(k, "bf16", "cuda:0")
    pairs = torch.tensor([[-1, 0], [6, 1], [2, 4], [1, 3]], dtype=torch.int32).cuda()
    pa.pa_swap_blocks(pairs, dk, dk, tk, tv)
    torch.cuda.synchronize()
    got = gd.to_numpy(tk, "bf16")
    assert np.array_equal(got[:3], h[:3]) and np.array_equal(got[3], k[1])


def _llama():
    w = W.llama3_8b_decode()
    gc = _gd().GpuCache(w).run()
    return w, gc


def test_swap_out_and_in_round_trip_is_bit_exact():
    """Swap the two longest sequences out, let another sequence take and
    overwrite the released blocks, decode the rest (against the oracle),
    swap them back into other blocks: the full decode is bit-identical."""
    import torch
    import paged_kv_cache_338_amd as pa
    w, gc = _llama()
    gd = _gd()
    maxb = 300
    out0 = gd.to_numpy(gc.decode(max_blocks=maxb), "bf16")
    nh = 512
    gc.alloc.add_host_pool(nh, np.random.default_rng(5).permutation(nh))
    shape = (nh, w.num_kv_heads, w.block_size, w.head_dim)
    hk = torch.empty(shape, dtype=torch.bfloat16).pin_memory()
    hv = torch.empty(shape, dtype=torch.bfloat16).pin_memory()
    free0 = gc.alloc.num_free()
    moved = 0
    for s in (4, 6):
        pairs = gc.alloc.seq_swap_out(s)
        moved += len(pairs)
        pa.pa_swap_blocks(torch.from_numpy(pairs).cuda(), gc.k_cache, gc.v_cache, hk, hv)
    assert gc.alloc.num_free() == free0 + moved and gc.alloc.num_free_host() == nh - moved
    # Another sequence takes (and overwrites) the released blocks.
    gc.alloc.seq_create(99)
    n_tok = gc.alloc.num_free() * w.block_size
    slots, _ = gc.alloc.seq_reserve([99], [n_tok])
    junk = torch.full((n_tok, w.num_kv_heads, w.head_dim), 3.0, dtype=torch.bfloat16).cuda()
    pa.pa_cache_append(junk, junk, torch.from_numpy(slots.copy()).cuda(), gc.k_cache, gc.v_cache)
    torch.cuda.synchronize()
    rest = [0, 1, 2, 3, 5, 7]
    t, l = gc.alloc.build_block_tables(rest, maxb)
    got = gc.decode(q=w.q[rest], tables=t, lens=l)
    oc = OracleCache(w).run()
    want = oc.decode()[rest]
    parity_log.within(gd.widen_out(got, "bf16"), want, 2e-2, "bf16")
    # Make room, swap back in (other device blocks), decode everything.
    gc.alloc.seq_free(99)
    for s in (6, 4):
        pairs = gc.alloc.seq_swap_in(s)
        pa.pa_swap_blocks(torch.from_numpy(pairs).cuda(), hk, hv, gc.k_cache, gc.v_cache)
    torch.cuda.synchronize()
    assert not gc.alloc.seq_is_swapped(4) and gc.alloc.num_free_host() == nh
    out1 = gd.to_numpy(gc.decode(max_blocks=maxb), "bf16")
    assert np.array_equal(out1, out0)


def test_drop_and_recompute_is_bit_exact():
    """Drop sequence 2's blocks, let another sequence take them, rebuild the
    sequence from its tokens' K/V rows (the prefill pass writes them again):
    decode output is bit-identical to before."""
    import torch
    import paged_kv_cache_338_amd as pa
    w, gc = _llama()
    gd = _gd()
    out0 = gd.to_numpy(gc.decode(max_blocks=300), "bf16")
    rows = [op[3] for op in w.script if op[0] == "reserve" and list(op[1]) == [2]]
    rows = np.concatenate(rows)
    gc.alloc.seq_free(2)
    gc.alloc.seq_create(50)
    gc.alloc.seq_reserve([50], [700])
    gc.alloc.seq_create(2)
    slots, _ = gc.alloc.seq_reserve([2], [len(rows)])
    idx = torch.from_numpy(rows.astype(np.int64)).cuda()
    pa.pa_cache_append(gc.k_rows.index_select(0, idx).contiguous(),
                       gc.v_rows.index_select(0, idx).contiguous(),
                       torch.from_numpy(slots.copy()).cuda(), gc.k_cache, gc.v_cache)
    torch.cuda.synchronize()
    out1 = gd.to_numpy(gc.decode(max_blocks=300), "bf16")
    assert np.array_equal(out1, out0)


def test_swap_binding_rejects_bad_arguments():
    import torch
    import paged_kv_cache_338_amd as pa
    dk = torch.zeros((4, 2, 8, 64), dtype=torch.bfloat16).cuda()
    host_unpinned = torch.zeros((4, 2, 8, 64), dtype=torch.bfloat16)
    pairs = torch.zeros((1, 2), dtype=torch.int32).cuda()
    with pytest.raises(ValueError):
        pa.pa_swap_blocks(pairs, dk, dk, host_unpinned, host_unpinned)
    other = torch.zeros((4, 2, 8, 128), dtype=torch.bfloat16).cuda()
    with pytest.raises(ValueError):
        pa.pa_swap_blocks(pairs, dk, dk, other, other)
