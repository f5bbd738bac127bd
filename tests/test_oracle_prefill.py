"""Oracle prefill (multi-query, causal) attention: pinned by the decode
oracle (one query token), a dense masked formulation, chunking invariance,
closed forms and brute force, with planted mistakes caught."""

import numpy as np
import pytest

from oracle import attention as oatt
from oracle import prefill as opf


def _random_case(seed, lengths, nq, H_q=4, H_kv=2, D=16, bs=4, dtype="f32", spare=3):
    """Random pools with blocks shuffled; sequence b holds lengths[b] tokens
    and its last nq[b] are the query tokens."""
    rng = np.random.default_rng(seed)
    nblk = [-(-L // bs) for L in lengths]
    nb = sum(nblk) + spare
    perm = rng.permutation(nb)
    tables = np.full((len(lengths), max(max(nblk), 1)), -1, np.int64)
    k = rng.standard_normal((nb, H_kv, bs, D)).astype(np.float32)
    v = rng.standard_normal((nb, H_kv, bs, D)).astype(np.float32)
    if dtype == "bf16":
        from workloads import round_to_bf16_bits
        k, v = round_to_bf16_bits(k), round_to_bf16_bits(v)
    c = 0
    for b, n in enumerate(nblk):
        tables[b, :n] = perm[c:c + n]
        c += n
    qs = np.concatenate([[0], np.cumsum(nq)]).astype(np.int64)
    q = rng.standard_normal((int(qs[-1]), H_q, D)).astype(np.float32)
    if dtype == "bf16":
        from workloads import round_to_bf16_bits
        q = round_to_bf16_bits(q)
    return q, k, v, tables, np.array(lengths), qs, bs


def _contiguous(k, v, tables, lens, bs):
    ks, vs = [], []
    for b, L in enumerate(lens):
        pos = np.arange(L)
        phys = tables[b, pos // bs]
        ks.append(k[phys, :, pos % bs, :])
        vs.append(v[phys, :, pos % bs, :])
    return ks, vs


def test_one_query_token_is_decode():
    q, k, v, t, lens, qs, bs = _random_case(1, [7, 16, 33, 1], [1, 1, 1, 1])
    got = opf.paged_prefill(q, k, v, t, lens, qs, bs, 0.3, "f32")
    want = oatt.paged_decode(q, k, v, t, lens, bs, 0.3, "f32")
    np.testing.assert_allclose(got, want, atol=1e-14, rtol=0)


@pytest.mark.parametrize("seed,lengths,nq", [(2, [9, 20, 5], [9, 4, 1]), (3, [31, 8], [12, 8]),
                                             (4, [64, 17, 3, 40], [16, 17, 2, 40])])
def test_matches_dense_masked_formulation(seed, lengths, nq):
    q, k, v, t, lens, qs, bs = _random_case(seed, lengths, nq)
    got = opf.paged_prefill(q, k, v, t, lens, qs, bs, 0.25, "f32")
    ks, vs = _contiguous(k, v, t, lens, bs)
    want = opf.dense_causal_prefill(q, ks, vs, qs, 0.25, "f32")
    np.testing.assert_allclose(got, want, atol=1e-12, rtol=0)


def test_brute_force_agrees():
    q, k, v, t, lens, qs, bs = _random_case(5, [6, 3], [4, 3], D=8)
    got = opf.paged_prefill(q, k, v, t, lens, qs, bs, 0.5, "f32")
    want = opf.brute_force_prefill(q, k, v, t, lens, qs, bs, 0.5, "f32")
    np.testing.assert_allclose(got, want, atol=1e-13, rtol=0)


def test_chunked_prefill_equals_whole_prompt():
    # One prompt of 37 tokens, prefilled at once or in chunks of 10, 1, 20,
    # 6: each chunk's queries see the prefix filled so far plus themselves.
    q, k, v, t, lens, qs, bs = _random_case(6, [37], [37])
    whole = opf.paged_prefill(q, k, v, t, lens, qs, bs, 0.2, "f32")
    done = 0
    for chunk in (10, 1, 20, 6):
        part = opf.paged_prefill(q[done:done + chunk], k, v, t, [done + chunk], [0, chunk], bs,
                                 0.2, "f32")
        np.testing.assert_allclose(part, whole[done:done + chunk], atol=1e-13, rtol=0)
        done += chunk


def test_first_prompt_token_returns_its_value_and_two_token_closed_form():
    q, k, v, t, lens, qs, bs = _random_case(7, [2], [2], H_q=2, H_kv=1, D=4)
    out = opf.paged_prefill(q, k, v, t, lens, qs, bs, 0.7, "f32")
    v0 = v[t[0, 0], 0, 0].astype(np.float64)
    v1 = v[t[0, 0], 0, 1].astype(np.float64)
    k0 = k[t[0, 0], 0, 0].astype(np.float64)
    k1 = k[t[0, 0], 0, 1].astype(np.float64)
    for h in range(2):
        np.testing.assert_array_equal(out[0, h], v0)  # one key: its value exactly
        qh = q[1, h].astype(np.float64)
        a = 1.0 / (1.0 + np.exp(0.7 * (qh @ k1 - qh @ k0)))  # weight of token 0
        np.testing.assert_allclose(out[1, h], a * v0 + (1 - a) * v1, atol=1e-14, rtol=0)


def test_physical_relabelling_is_invisible():
    q, k, v, t, lens, qs, bs = _random_case(8, [13, 22], [5, 22], dtype="bf16")
    want = opf.paged_prefill(q, k, v, t, lens, qs, bs, 0.3, "bf16")
    rng = np.random.default_rng(9)
    pi = rng.permutation(k.shape[0])
    k2, v2 = np.empty_like(k), np.empty_like(v)
    k2[pi], v2[pi] = k, v
    t2 = np.where(t >= 0, pi[np.maximum(t, 0)], -1)
    np.testing.assert_array_equal(opf.paged_prefill(q, k2, v2, t2, lens, qs, bs, 0.3, "bf16"), want)


def test_rejects_more_queries_than_tokens():
    q, k, v, t, lens, qs, bs = _random_case(10, [3], [3])
    with pytest.raises(ValueError):
        opf.paged_prefill(q, k, v, t, [2], qs, bs, 0.3, "f32")


def test_flop_count():
    # Prompt of 3 (whole): rows see 1, 2, 3 keys -> 6 pairs; chunk of 2 on
    # a context of 5: rows see 4 and 5 keys -> 9 pairs.
    assert opf.prefill_flops([3, 5], [0, 3, 5], 2, 8) == (6 + 9) * 2 * 4 * 8


# ---- planted mistakes: each must break at least one pin above --------------
def _variant(mistake):
    def fn(q, k_cache, v_cache, block_tables, context_lens, query_start, block_size, scale, dtype):
        qf = oatt.widen(q, dtype)
        T, H_q, D = qf.shape
        H_kv = k_cache.shape[1]
        G = H_q // H_kv
        out = np.zeros((T, H_q, D))
        for b in range(len(context_lens)):
            L, n = int(context_lens[b]), int(query_start[b + 1] - query_start[b])
            pos = np.arange(L)
            phys = np.asarray(block_tables)[b, pos // block_size]
            for kvh in range(H_kv):
                K = oatt.widen(k_cache[phys, kvh, pos % block_size], dtype)
                V = oatt.widen(v_cache[phys, kvh, pos % block_size], dtype)
                for i in range(n):
                    p = i if mistake == "position_from_zero" else L - n + i
                    end = p if mistake == "strict_mask" else p + 1
                    end = L if mistake == "no_mask" else end
                    for g in range(G):
                        h = kvh * G + g
                        s = scale * (K[:max(end, 1)] @ qf[query_start[b] + i, h])
                        w = np.exp(s - s.max())
                        out[query_start[b] + i, h] = (w @ V[:max(end, 1)]) / w.sum()
        return out
    return fn


@pytest.mark.parametrize("mistake", ["position_from_zero", "strict_mask", "no_mask"])
def test_planted_mistakes_are_caught(mistake):
    bad = _variant(mistake)
    q, k, v, t, lens, qs, bs = _random_case(4, [64, 17, 3, 40], [16, 17, 2, 40])
    ks, vs = _contiguous(k, v, t, lens, bs)
    want = opf.dense_causal_prefill(q, ks, vs, qs, 0.25, "f32")
    got = bad(q, k, v, t, lens, qs, bs, 0.25, "f32")
    assert not np.allclose(got, want, atol=1e-9)


def test_correct_variant_passes():
    good = _variant("none")
    q, k, v, t, lens, qs, bs = _random_case(4, [64, 17, 3, 40], [16, 17, 2, 40])
    ks, vs = _contiguous(k, v, t, lens, bs)
    want = opf.dense_causal_prefill(q, ks, vs, qs, 0.25, "f32")
    np.testing.assert_allclose(good(q, k, v, t, lens, qs, bs, 0.25, "f32"), want, atol=1e-12)
