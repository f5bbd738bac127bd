"""HIP path vs the CPU oracle on the same seeded inputs (needs a gfx950 GPU).

Append, block copy, block tables and allocator state must be bit-exact;
attention outputs within max-abs 1e-4 (fp32 pools) or 2e-2 (bf16 pools,
N(0, 1) inputs).  Pools start NaN-poisoned, so any read of an unwritten or
masked slot shows up as a non-finite or wrong output.
"""

import functools
import os

import numpy as np
import pytest

import parity_log
import workloads as W
from oracle import attention as oatt
from oracle import cache_ops as ocops
from oracle_driver import OracleCache

pytestmark = pytest.mark.gpu

# fp16: probabilities rounded to fp16 move each normalised weight by at most
# 2^-11 relative, so the output by at most 2^-11 max|v - out| (< 10 for
# N(0, 1) values: 4.9e-3), plus 2^-11 |out| for the final rounding.
TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 6e-3}


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


def assert_close(w, got_t, want, tol=None):
    got = _gd().widen_out(got_t, w.dtype)
    assert got.shape == want.shape
    assert np.isfinite(got).all()
    return parity_log.within(got, want, TOL[w.dtype] if tol is None else tol, w.dtype, w.name)


def assert_pools_equal(w, gc, oc):
    gd = _gd()
    assert np.array_equal(gd.to_numpy(gc.k_cache, w.dtype).view(np.uint8),
                          np.ascontiguousarray(oc.k_cache).view(np.uint8))
    assert np.array_equal(gd.to_numpy(gc.v_cache, w.dtype).view(np.uint8),
                          np.ascontiguousarray(oc.v_cache).view(np.uint8))


def run_both(w):
    oc = OracleCache(w).run()
    gc = _gd().GpuCache(w).run()
    for (so, po), (sg, pg) in zip([x[1] for x in oc.log if x[0] == "reserve"], gc.log):
        assert np.array_equal(so, sg) and np.array_equal(po, pg)
    to, lo = oc.tables()
    tg, lg = gc.tables(to.shape[1])
    assert np.array_equal(to, tg) and np.array_equal(lo, lg)
    return oc, gc


def test_tiny_ref():
    w = W.tiny_ref()
    oc, gc = run_both(w)
    assert_pools_equal(w, gc, oc)
    want = oc.decode()
    assert_close(w, gc.decode(), want)
    np.testing.assert_allclose(want, oc.contiguous(), atol=1e-12, rtol=0)


def test_llama3_8b_batch_and_one_step():
    w = W.llama3_8b_decode()
    oc, gc = run_both(w)
    assert_pools_equal(w, gc, oc)
    assert_close(w, gc.decode(), oc.decode())
    # One decode step: reserve a token per sequence, append it, decode L + 1.
    rows_k = np.concatenate([w.k_rows, w.notes["new_k"]])
    rows_v = np.concatenate([w.v_rows, w.notes["new_v"]])
    w.k_rows, w.v_rows = rows_k, rows_v
    gc.k_rows = _gd().to_torch(rows_k, w.dtype, gc.device)
    gc.v_rows = _gd().to_torch(rows_v, w.dtype, gc.device)
    n0 = len(rows_k) - w.batch
    step = [("reserve", w.seq_ids, [1] * w.batch, np.arange(n0, n0 + w.batch))]
    oc.run(step)
    gc.run(step)
    assert_pools_equal(w, gc, oc)
    to, lo = oc.tables()
    assert lo.tolist() == [L + 1 for L in W.LLAMA3_8B_BATCH]
    assert_close(w, gc.decode(), oc.decode())


def test_serving_batch():
    w = W.serving_batch()
    oc, gc = run_both(w)
    assert_pools_equal(w, gc, oc)
    assert_close(w, gc.decode(), oc.decode())


@functools.lru_cache(maxsize=1)
def _sweep_values():
    return W.block_size_sweep(8)


@pytest.mark.parametrize("bs", W.BLOCK_SIZE_SWEEP)
def test_block_size_sweep(bs):
    base = _sweep_values()
    w = W.block_size_sweep(bs, with_values=False)
    w.q, w.k_rows, w.v_rows = base.q, base.k_rows, base.v_rows
    oc, gc = run_both(w)
    assert_pools_equal(w, gc, oc)
    assert_close(w, gc.decode(), oc.decode())


@pytest.mark.parametrize("prefix_len,pairs", [(2056, 127), (2048, 0)])
def test_prefix_sharing_copy_on_write(prefix_len, pairs):
    w = W.prefix_sharing(prefix_len=prefix_len)
    oc, gc = run_both(w)
    assert len(gc.log[-1][1]) == pairs
    assert_pools_equal(w, gc, oc)
    assert_close(w, gc.decode(), oc.decode())


def _small(seed, lengths, G=4, H_kv=2, D=128, bs=16, dtype="bf16", spare=3):
    """A tiny hand-sized workload (same generator recipe, arbitrary shape)."""
    rng = np.random.default_rng(seed)
    nb = sum(-(-L // bs) for L in lengths) + spare
    free_order = rng.permutation(nb).astype(np.int32)
    mk = lambda *s: W._normal(rng, s, dtype)
    q = mk(len(lengths), G * H_kv, D)
    k = mk(max(1, sum(lengths)), H_kv, D)
    v = mk(max(1, sum(lengths)), H_kv, D)
    script, logical = W._sequential_script(lengths)
    return W.Workload("small", seed, G * H_kv, H_kv, D, bs, dtype, 1.0 / np.sqrt(D), nb,
                      free_order, q, k, v, script, list(range(len(lengths))), logical)


SHAPES = [
    # (G, H_kv, D, bs, dtype, lengths)
    (4, 2, 128, 16, "bf16", [1, 15, 16, 17, 31, 32, 33, 200]),
    (1, 3, 128, 16, "bf16", [5, 40, 100]),
    (2, 2, 64, 8, "bf16", [7, 8, 9, 130]),
    (8, 1, 128, 32, "bf16", [1, 33, 64, 65, 500]),
    (16, 1, 128, 16, "bf16", [300, 3]),
    (3, 2, 128, 16, "bf16", [50, 51]),
    (4, 2, 128, 4, "bf16", [3, 4, 5, 77]),
    (4, 2, 128, 1, "bf16", [1, 2, 19]),
    (4, 2, 128, 128, "bf16", [1, 127, 128, 129, 400]),
    (4, 2, 128, 256, "bf16", [255, 256, 257]),
    (2, 2, 64, 4, "f32", [1, 4, 5, 63, 64]),
    (4, 2, 128, 16, "f32", [16, 17, 100]),
    (4, 1, 64, 2, "f32", [9, 3]),
    (3, 2, 128, 32, "f32", [1, 31, 32, 33, 300]),
    (8, 1, 128, 128, "f32", [1, 127, 128, 129, 400]),
    (16, 1, 128, 256, "f32", [255, 256, 257, 600]),
    (3, 2, 64, 16, "f32", [17, 90]),
    (8, 1, 128, 16, "f32", [1, 16, 17, 250]),
    (16, 1, 64, 32, "f32", [31, 33, 200]),
    (4, 2, 128, 16, "f16", [1, 15, 16, 17, 31, 32, 33, 200]),
    (8, 1, 64, 8, "f16", [5, 130, 64]),
    (4, 2, 128, 4, "f16", [3, 4, 77]),
    (16, 1, 128, 32, "f16", [300, 1]),
    (4, 8, 128, 16, "f16", [128, 700, 1500, 300]),
    (3, 2, 128, 16, "f16", [50, 51, 1, 333]),
    (3, 1, 64, 32, "f16", [31, 32, 33, 97]),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"G{s[0]}_H{s[1]}_D{s[2]}_bs{s[3]}_{s[4]}"
                                               for s in SHAPES])
def test_shapes(shape):
    G, H_kv, D, bs, dtype, lengths = shape
    w = _small(17, lengths, G, H_kv, D, bs, dtype)
    oc, gc = run_both(w)
    assert_pools_equal(w, gc, oc)
    assert_close(w, gc.decode(), oc.decode())
    # A wider table (padding with -1 past each sequence) changes nothing.
    to, lo = oc.tables()
    wide = np.full((to.shape[0], to.shape[1] + 5), -1, np.int32)
    wide[:, :to.shape[1]] = to
    assert_close(w, gc.decode(tables=wide, lens=lo), oc.decode())


@pytest.mark.parametrize("case", ["llama", "prefix2056", "bs4", "f32_g8", "f16_bs8"])
def test_kv_load_policy_does_not_change_the_result(case):
    """pa_decode with non-temporal K/V loads (the default) and with cached
    loads (PA_TUNE_DECODE_KV_CACHED = 1): the same kernel arithmetic, so the
    outputs are bit-identical, and both match the oracle."""
    import paged_kv_cache_338_amd as pa
    if case == "llama":
        w = W.llama3_8b_decode()
    elif case == "prefix2056":
        w = W.prefix_sharing(prefix_len=2056)
    elif case == "bs4":
        w = _small(41, [3, 4, 5, 77, 300], 4, 2, 128, 4, "bf16")
    elif case == "f32_g8":
        w = _small(42, [1, 16, 17, 250], 8, 1, 128, 16, "f32")
    else:
        w = _small(43, [5, 130, 64], 8, 1, 64, 8, "f16")
    oc, gc = run_both(w)
    want = oc.decode()
    outs = []
    for cached in (0, 1):
        with pa.tuning(pa.PA_TUNE_DECODE_KV_CACHED, cached):
            out = gc.decode()
        assert_close(w, out, want)
        outs.append(_gd().to_numpy(out, w.dtype))
    assert np.array_equal(outs[0], outs[1])


def _direct_case(seed, lens, H_kv, G, D, bs, dtype):
    """Pools, tables and queries built directly: each sequence's blocks a
    shuffled slice of the pool, only its own token slots hold values, every
    other slot NaN."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, np.int32)
    B = len(lens)
    nblk = -(-lens // bs)
    nb = int(nblk.sum()) + 1
    perm = rng.permutation(nb).astype(np.int32)
    tables = np.full((B, max(1, int(nblk.max()))), -1, np.int32)
    starts = np.concatenate([[0], np.cumsum(nblk)])
    for b in range(B):
        tables[b, :nblk[b]] = perm[starts[b]:starts[b + 1]]
    seq = np.repeat(np.arange(B), lens)
    pos = np.concatenate([np.arange(L) for L in lens])
    blk, off = tables[seq, pos // bs], pos % bs
    store = np.uint16 if dtype == "bf16" else np.float32
    poison = np.array(0x7FC0, np.uint16) if dtype == "bf16" else np.float32(np.nan)
    k = np.full((nb, H_kv, bs, D), poison, store)
    v = np.full((nb, H_kv, bs, D), poison, store)
    k[blk, :, off] = W._normal(rng, (len(seq), H_kv, D), dtype)
    v[blk, :, off] = W._normal(rng, (len(seq), H_kv, D), dtype)
    q = W._normal(rng, (B, G * H_kv, D), dtype)
    return q, k, v, tables, lens


def _direct_decode(q, k, v, tables, lens, bs, scale, dtype):
    import torch
    import paged_kv_cache_338_amd as pa
    gd, dev = _gd(), "cuda:0"
    qd = gd.to_torch(q, dtype, dev)
    out = torch.empty_like(qd)
    pa.pa_decode(qd, gd.to_torch(k, dtype, dev), gd.to_torch(v, dtype, dev),
                 torch.from_numpy(tables).to(dev), torch.from_numpy(lens).to(dev), bs, scale, out)
    torch.cuda.synchronize()
    return gd.widen_out(out, dtype)


def test_one_context_of_131072_tokens():
    """One 131,072-token sequence beside two short ones, 8 query / 2 KV heads,
    head 128: each of its two segments spans about 500 of the grid's 1,024
    waves, so the merge combines more contributors than one pass holds."""
    q, k, v, tables, lens = _direct_case(131072, [131072, 3, 700], 2, 4, 128, 16, "bf16")
    scale = 1.0 / np.sqrt(128)
    got = _direct_decode(q, k, v, tables, lens, 16, scale, "bf16")
    want = oatt.paged_decode(q, k, v, tables, lens, 16, scale, "bf16")
    assert np.isfinite(got).all()
    parity_log.within(got, want, TOL["bf16"], "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_maximum_batch_of_8192_sequences(dtype):
    """The largest batch pa_decode takes (8,192 sequences): its lengths
    snapshot needs more than 64 KiB of LDS (the launch raises the kernel's
    LDS limit), and the merge grid has 8,192 x H_kv x G workgroups.  Lengths
    0..40 (some empty), one KV head, head 64, 16-token blocks, blocks
    shuffled over the pool; every other slot NaN.  Tables and pools are
    built directly (the allocator's own tests cover the allocator)."""
    rng = np.random.default_rng(8192 + (dtype == "f32"))
    lens = rng.integers(0, 41, 8192).astype(np.int32)
    q, k, v, tables, lens = _direct_case(8192 + (dtype == "f32"), lens, 1, 4, 64, 16, dtype)
    scale = 1.0 / 8
    want = oatt.paged_decode(q, k, v, tables, lens, 16, scale, dtype)
    got = _direct_decode(q, k, v, tables, lens, 16, scale, dtype)
    assert np.isfinite(got).all()
    assert np.array_equal(got[lens == 0], np.zeros_like(got[lens == 0]))
    parity_log.within(got, want, TOL[dtype], dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_token_returns_v_exactly(dtype):
    w = _small(5, [1, 1, 1], G=4, H_kv=2, D=128, bs=16, dtype=dtype)
    oc, gc = run_both(w)
    got = _gd().to_numpy(gc.decode(), dtype)
    for b in range(3):
        row = w.v_rows[w.logical_rows[b][0]]
        for h in range(8):
            assert np.array_equal(got[b, h], row[h // 4]), (b, h)


def test_zero_length_sequences_give_zeros():
    w = _small(6, [0, 20, 0, 3], G=4, H_kv=2, D=128, bs=16)
    oc, gc = run_both(w)
    out = gc.decode()
    want = oc.decode()
    assert_close(w, out, want)
    got = _gd().widen_out(out, w.dtype)
    assert np.array_equal(got[0], np.zeros_like(got[0]))
    assert np.array_equal(got[2], np.zeros_like(got[2]))


def test_physical_relabelling_is_bit_identical():
    import torch
    w = W.llama3_8b_decode()
    gc = _gd().GpuCache(w).run()
    tables, lens = gc.tables()
    base = gc.decode(tables=tables, lens=lens)
    perm = np.random.default_rng(99).permutation(w.num_blocks)
    pt = torch.from_numpy(perm).to(gc.device)
    k2 = torch.empty_like(gc.k_cache)
    v2 = torch.empty_like(gc.v_cache)
    k2[pt] = gc.k_cache
    v2[pt] = gc.v_cache
    gc.k_cache, gc.v_cache = k2, v2
    t2 = np.where(tables >= 0, perm[np.maximum(tables, 0)], -1).astype(np.int32)
    out = gc.decode(tables=t2, lens=lens)
    assert torch.equal(out.view(torch.int16), base.view(torch.int16))


@pytest.mark.parametrize("wgs", [1, 3, 8, 97, 256, 264, 1024])
def test_grid_size_does_not_change_the_result(wgs):
    # The grid splits the flat tile list into equal shares; a share boundary
    # inside a (KV head, sequence) segment leaves partials that the last
    # workgroup to arrive merges, from its own L2 when every piece ran on
    # one XCD, else at device scope (grids that are not a multiple of 8 deal
    # consecutive shares to different XCDs).  Any grid size must give the
    # same result.
    import paged_kv_cache_338_amd as pa
    w = W.llama3_8b_decode()
    oc, gc = run_both(w)
    want = oc.decode()
    with pa.tuning(pa.PA_TUNE_DECODE_WORKGROUPS, wgs):
        got = gc.decode()
    assert_close(w, got, want)


def test_copy_blocks_direct_bit_exact():
    import torch
    import paged_kv_cache_338_amd as pa
    gd = _gd()
    rng = np.random.default_rng(8)
    for dtype, shape in (("bf16", (40, 8, 16, 128)), ("f32", (12, 2, 4, 64))):
        k = W._normal(rng, shape, dtype)
        v = W._normal(rng, shape, dtype)
        pairs = np.array([[3, 7], [0, 5], [9, 1]], np.int32)
        kd, vd = gd.to_torch(k, dtype, "cuda:0"), gd.to_torch(v, dtype, "cuda:0")
        pa.pa_copy_blocks(torch.from_numpy(pairs).cuda(), kd, vd)
        ocops.copy_blocks(k, v, pairs)
        assert np.array_equal(gd.to_numpy(kd, dtype).view(np.uint8), k.view(np.uint8))
        assert np.array_equal(gd.to_numpy(vd, dtype).view(np.uint8), v.view(np.uint8))


def test_append_skips_negative_slots_and_oracle_agrees():
    import torch
    import paged_kv_cache_338_amd as pa
    gd = _gd()
    rng = np.random.default_rng(9)
    shape = (6, 2, 8, 64)
    k = np.full(shape, W.POISON_BITS["bf16"], np.uint16)
    v = k.copy()
    rows_k = W._normal(rng, (5, 2, 64), "bf16")
    rows_v = W._normal(rng, (5, 2, 64), "bf16")
    slots = np.array([47, -1, 0, 8, -5], np.int64)
    kd, vd = gd.to_torch(k, "bf16", "cuda:0"), gd.to_torch(v, "bf16", "cuda:0")
    pa.pa_cache_append(gd.to_torch(rows_k, "bf16", "cuda:0"), gd.to_torch(rows_v, "bf16", "cuda:0"),
                       torch.from_numpy(slots).cuda(), kd, vd)
    ocops.cache_append(k, v, rows_k, rows_v, slots, 8)
    assert np.array_equal(gd.to_numpy(kd, "bf16"), k)
    assert np.array_equal(gd.to_numpy(vd, "bf16"), v)


def test_python_binding_rejects_bad_arguments():
    import torch
    import paged_kv_cache_338_amd as pa
    kc = torch.zeros(4, 2, 16, 128, dtype=torch.bfloat16, device="cuda:0")
    q = torch.zeros(1, 4, 128, dtype=torch.bfloat16, device="cuda:0")
    t = torch.zeros(1, 2, dtype=torch.int32, device="cuda:0")
    l = torch.ones(1, dtype=torch.int32, device="cuda:0")
    with pytest.raises(pa.PagedAttentionError):
        pa.pa_decode(q, kc, kc, t, l, 8, 1.0, torch.empty_like(q))  # wrong block size
    with pytest.raises(TypeError):
        pa.pa_decode(q, kc, kc, t.long(), l, 16, 1.0, torch.empty_like(q))


def test_workspace_zero_filled_once_serves_every_call():
    # Only the arrival counters must start at zero (they follow the
    # published partial results, B * H_kv 64-bit words); every call puts them
    # back to zero and writes each published piece before it is read, so
    # garbage elsewhere is harmless and one workspace serves any number of
    # calls and grid sizes, with the counters zero after each.
    import torch
    import paged_kv_cache_338_amd as pa
    w = W.llama3_8b_decode()
    oc, gc = run_both(w)
    want = oc.decode()
    tables, lens = gc.tables()
    qd = _gd().to_torch(w.q, w.dtype, gc.device)
    td = torch.from_numpy(tables).to(gc.device)
    ld = torch.from_numpy(lens).to(gc.device)
    ws = pa.decode_workspace(gc.k_cache, w.batch, w.num_q_heads, tables.shape[1])
    nctr = -(-w.batch * w.num_kv_heads * 8 // 256) * 256
    ws.fill_(0xFF)
    ws[-nctr:].zero_()
    for wgs in (256, 1000, 37, 256, 1, 512):
        with pa.tuning(pa.PA_TUNE_DECODE_WORKGROUPS, wgs):
            out = torch.empty_like(qd)
            pa.pa_decode(qd, gc.k_cache, gc.v_cache, td, ld, w.block_size, w.scale, out,
                         workspace=ws)
        torch.cuda.synchronize()
        assert_close(w, out, want)
        assert not ws[-nctr:].any(), wgs


def test_workspace_serves_smaller_batches_between_larger_ones():
    # One zero fill serves calls of any batch size up to the one the
    # workspace was sized for: a call with fewer sequences uses a prefix of
    # the counters and leaves it at zero, and the published pieces never
    # overlap the counters (regression: the counters used to come first, so
    # a larger batch found the pieces of a smaller one there).
    import torch
    import paged_kv_cache_338_amd as pa
    w = W.llama3_8b_decode()
    oc, gc = run_both(w)
    want = oc.decode()
    tables, lens = gc.tables()
    qd = _gd().to_torch(w.q, w.dtype, gc.device)
    td = torch.from_numpy(tables).to(gc.device)
    ld = torch.from_numpy(lens).to(gc.device)
    ws = pa.decode_workspace(gc.k_cache, w.batch, w.num_q_heads, tables.shape[1])
    for sl in (slice(0, 8), slice(2, 5), slice(0, 8), slice(6, 8), slice(0, 1), slice(0, 8)):
        q, t, l = qd[sl].contiguous(), td[sl].contiguous(), ld[sl].contiguous()
        out = torch.empty_like(q)
        pa.pa_decode(q, gc.k_cache, gc.v_cache, t, l, w.block_size, w.scale, out, workspace=ws)
        torch.cuda.synchronize()
        assert_close(w, out, want[sl])


def test_graph_replay_matches_eager_and_reads_lengths_at_run_time():
    # pa_cache_append and pa_decode enqueue only kernel launches (no memset,
    # no allocation), so a captured HIP graph replays them; the decode reads
    # the lengths from device memory at run time, so a replay after the
    # lengths change follows them.  Each replay is checked, with eager work
    # and synchronisations in between.
    import torch
    import paged_kv_cache_338_amd as pa
    w = W.llama3_8b_decode()
    oc, gc = run_both(w)
    tables, lens = gc.tables()
    qd = _gd().to_torch(w.q, w.dtype, gc.device)
    td = torch.from_numpy(tables).to(gc.device)
    ld = torch.from_numpy(lens).to(gc.device)
    # Re-append the last token of every sequence (same rows, same slots).
    last = np.array([len(r) - 1 for r in w.logical_rows])
    rows = np.array([w.logical_rows[b][last[b]] for b in range(w.batch)])
    slots = np.array([tables[b, last[b] // w.block_size] * w.block_size + last[b] % w.block_size
                      for b in range(w.batch)], np.int64)
    kr = gc.k_rows.index_select(0, torch.from_numpy(rows).to(gc.device)).contiguous()
    vr = gc.v_rows.index_select(0, torch.from_numpy(rows).to(gc.device)).contiguous()
    sd = torch.from_numpy(slots).to(gc.device)
    ws = pa.decode_workspace(gc.k_cache, w.batch, w.num_q_heads, tables.shape[1])
    out_e = torch.empty_like(qd)
    pa.pa_decode(qd, gc.k_cache, gc.v_cache, td, ld, w.block_size, w.scale, out_e, workspace=ws)
    torch.cuda.synchronize()
    want = oc.decode()
    assert_close(w, out_e, want)

    out_g = torch.empty_like(qd)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            pa.pa_cache_append(kr, vr, sd, gc.k_cache, gc.v_cache)
            pa.pa_decode(qd, gc.k_cache, gc.v_cache, td, ld, w.block_size, w.scale, out_g,
                         workspace=ws)
    torch.cuda.synchronize()
    short = np.maximum(lens - 37, 1).astype(np.int32)
    want_short = oc.decode(tables=tables, lens=short)
    for rep in range(4):
        use_short = rep == 2
        ld.copy_(torch.from_numpy(short if use_short else lens))
        out_g.fill_(float("nan"))
        # eager work on the same workspace and stream between replays
        tmp = torch.empty_like(qd)
        pa.pa_decode(qd, gc.k_cache, gc.v_cache, td, ld, w.block_size, w.scale, tmp, workspace=ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), tmp.view(torch.int16)), rep
        assert_close(w, out_g, want_short if use_short else want)
    assert_pools_equal(w, gc, oc)
