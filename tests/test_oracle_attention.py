"""Oracle decode attention: pinned by closed forms, scipy, brute force and
invariants the pages state (paging leaves the attention arithmetic alone)."""

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle_pins as pins
import workloads as W
from oracle import attention as oatt
from oracle_driver import OracleCache


def test_two_token_closed_form():
    pins.check_two_token_closed_form(oatt.paged_decode)


def test_gqa_grouping():
    pins.check_gqa_grouping(oatt.paged_decode)


def test_single_token_is_v():
    pins.check_single_token_is_v(oatt.paged_decode)


def test_zero_query_mean():
    pins.check_zero_query_mean(oatt.paged_decode)


def test_against_scipy_softmax():
    pins.check_scaled_two_block_vs_scipy(oatt.paged_decode)


def test_brute_force_two_token_closed_form():
    pins.check_two_token_closed_form(oatt.brute_force_decode)
    pins.check_gqa_grouping(oatt.brute_force_decode)


def test_widen_bf16_exact():
    bits = np.array([0x3F80, 0xC000, 0x3F00, 0x0001, 0x7F7F, 0x8000], dtype=np.uint16)
    vals = oatt.widen(bits, "bf16")
    assert vals.tolist() == [1.0, -2.0, 0.5, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127, -0.0]
    with pytest.raises(TypeError):
        oatt.widen(np.zeros(2, np.float32), "bf16")


def test_equal_keys_give_mean_v_and_equal_values_give_v():
    rng = np.random.default_rng(5)
    bs, D, L = 4, 8, 9
    q = rng.standard_normal((1, 1, D)).astype(np.float32)
    kc = np.broadcast_to(rng.standard_normal(D).astype(np.float32), (3, 1, bs, D)).copy()
    vc = rng.standard_normal((3, 1, bs, D)).astype(np.float32)
    tab = np.array([[1, 2, 0]])
    out = oatt.paged_decode(q, kc, vc, tab, [L], bs, 0.5, "f32")
    rows = [vc[tab[0, p // bs], 0, p % bs].astype(np.float64) for p in range(L)]
    np.testing.assert_allclose(out[0, 0], np.mean(rows, axis=0), atol=1e-14, rtol=0)
    kc = rng.standard_normal((3, 1, bs, D)).astype(np.float32)
    c = rng.standard_normal(D).astype(np.float32)
    vc = np.broadcast_to(c, (3, 1, bs, D)).copy()
    out = oatt.paged_decode(q, kc, vc, tab, [L], bs, 0.5, "f32")
    np.testing.assert_allclose(out[0, 0], c.astype(np.float64), atol=1e-14, rtol=0)


def test_zero_context_gives_zeros():
    q = np.ones((2, 2, 4), np.float32)
    kc = np.full((2, 1, 2, 4), np.nan, np.float32)
    out = oatt.paged_decode(q, kc, kc, np.array([[0], [1]]), [0, 0], 2, 1.0, "f32")
    assert np.array_equal(out, np.zeros((2, 2, 4)))


def test_tiny_ref_three_ways():
    """Paged (through the table) == contiguous (scipy) == scalar brute force."""
    w = W.tiny_ref()
    oc = OracleCache(w).run()
    tables, lens = oc.tables()
    paged = oc.decode()
    cont = oc.contiguous()
    brute = oatt.brute_force_decode(w.q, oc.k_cache, oc.v_cache, tables, lens,
                                    w.block_size, w.scale, w.dtype)
    np.testing.assert_allclose(paged, cont, atol=1e-12, rtol=0)
    np.testing.assert_allclose(paged, brute, atol=1e-12, rtol=0)
    assert np.isfinite(paged).all()


def test_physical_relabelling_is_invisible():
    """Any permutation of physical block ids (contents moved, tables mapped)
    leaves the output bit-identical: only logical order matters."""
    w = W.tiny_ref()
    oc = OracleCache(w).run()
    tables, lens = oc.tables()
    base = oc.decode()
    perm = np.random.default_rng(11).permutation(w.num_blocks)
    k2 = np.empty_like(oc.k_cache)
    v2 = np.empty_like(oc.v_cache)
    k2[perm] = oc.k_cache
    v2[perm] = oc.v_cache
    t2 = np.where(tables >= 0, perm[np.maximum(tables, 0)], -1)
    out = oatt.paged_decode(w.q, k2, v2, t2, lens, w.block_size, w.scale, w.dtype)
    assert np.array_equal(out, base)


def _random_case(seed, B, G, H_kv, D, bs, max_len, dtype):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, max_len + 1, size=B)
    nblk = [-(-int(L) // bs) for L in lens]
    nb = sum(nblk) + 3
    perm = rng.permutation(nb)
    tables = np.full((B, max(1, max(nblk))), -1, np.int64)
    i = 0
    for b in range(B):
        tables[b, :nblk[b]] = perm[i:i + nblk[b]]
        i += nblk[b]
    if dtype == "bf16":
        mk = lambda *s: W.round_to_bf16_bits(rng.standard_normal(s).astype(np.float32))
    else:
        mk = lambda *s: rng.standard_normal(s).astype(np.float32)
    q = mk(B, G * H_kv, D)
    kc = mk(nb, H_kv, bs, D)
    vc = mk(nb, H_kv, bs, D)
    return q, kc, vc, tables, lens


@settings(max_examples=40, deadline=None)
@given(seed=st.integers(0, 10 ** 6), B=st.integers(1, 3), G=st.sampled_from([1, 2, 4]),
       H_kv=st.integers(1, 2), D=st.sampled_from([1, 3, 8]), bs=st.sampled_from([1, 2, 4, 8]),
       max_len=st.integers(0, 20), dtype=st.sampled_from(["f32", "bf16"]))
def test_paged_contiguous_brute_agree(seed, B, G, H_kv, D, bs, max_len, dtype):
    q, kc, vc, tables, lens = _random_case(seed, B, G, H_kv, D, bs, max_len, dtype)
    scale = 0.37
    paged = oatt.paged_decode(q, kc, vc, tables, lens, bs, scale, dtype)
    brute = oatt.brute_force_decode(q, kc, vc, tables, lens, bs, scale, dtype)
    ks = [np.stack([kc[tables[b, p // bs], :, p % bs] for p in range(lens[b])])
          if lens[b] else np.zeros((0, H_kv, D), kc.dtype) for b in range(B)]
    vs = [np.stack([vc[tables[b, p // bs], :, p % bs] for p in range(lens[b])])
          if lens[b] else np.zeros((0, H_kv, D), vc.dtype) for b in range(B)]
    cont = oatt.contiguous_decode(q, ks, vs, scale, dtype)
    np.testing.assert_allclose(paged, brute, atol=1e-12, rtol=0)
    np.testing.assert_allclose(paged, cont, atol=1e-12, rtol=0)


def test_f16_widening_and_rounding_pins():
    """IEEE binary16 bit patterns widen to their exact values, and the input
    generator rounds to nearest even (1/3 -> 0x3555, the float nearest)."""
    import workloads as W
    bits = np.array([0x3C00, 0xC000, 0x0001, 0x7BFF, 0x3555, 0x8000], np.uint16)
    got = oatt.widen(bits, "f16")
    assert got.tolist() == [1.0, -2.0, 2.0 ** -24, 65504.0, 1365 / 4096, -0.0]
    assert W.round_to_f16_bits(np.float32([1 / 3, 1.0, 65504.0, 2.0 ** -25 * 3]))[:3].tolist() == \
        [0x3555, 0x3C00, 0x7BFF]
    assert W.round_to_f16_bits(np.float32([2.0 ** -25 * 3]))[0] == 0x0002  # 1.5 ulp -> even (2)
    with pytest.raises(TypeError):
        oatt.widen(np.zeros(2, np.float16), "f16")
