"""Planted mistakes in copies of the oracle must trip at least one pin.

Each case patches one plausible error into the oracle (a wrong index, a
dropped term, a transposed operand, eager allocation, a wrong free order)
and checks that the pins catch it.  The mistakes live only in this file.
"""

import numpy as np
import pytest

import oracle_pins as pins
from oracle import attention as oatt
from oracle.allocator import BlockAllocator, OutOfBlocks


def _fails(check, *args):
    try:
        check(*args)
    except (AssertionError, IndexError, ValueError):
        return True
    return False


def _decode_variant(mistake):
    def fn(q, k_cache, v_cache, tables, lens, bs, scale, dtype):
        qf = oatt.widen(q, dtype)
        B, H_q, D = qf.shape
        H_kv = k_cache.shape[1]
        G = H_q // H_kv
        tables = np.asarray(tables)
        out = np.zeros((B, H_q, D))
        for b in range(B):
            L = int(lens[b])
            if L == 0:
                continue
            pos = np.arange(L)
            phys = tables[b, pos // bs]
            off = pos % bs
            if mistake == "offset_from_block":
                off = (pos // bs) % bs
            for h in range(H_q):
                kvh = h % H_kv if mistake == "gqa_modulo" else h // G
                K = oatt.widen(k_cache[phys, kvh, off, :], dtype)
                V = oatt.widen(v_cache[phys, kvh, off, :], dtype)
                if mistake == "k_for_v":
                    V = K
                s = K @ qf[b, h] if mistake == "no_scale" else scale * (K @ qf[b, h])
                if mistake == "sign":
                    s = -s
                w = np.exp(s - s.max())
                den = L if mistake == "mean_denominator" else w.sum()
                out[b, h] = (w @ V) / den
        return out
    return fn


DECODE_PINS = [pins.check_two_token_closed_form, pins.check_gqa_grouping,
               pins.check_single_token_is_v, pins.check_zero_query_mean,
               pins.check_scaled_two_block_vs_scipy]


@pytest.mark.parametrize("mistake", ["offset_from_block", "gqa_modulo", "k_for_v", "no_scale",
                                     "sign", "mean_denominator"])
def test_decode_mistake_is_caught(mistake):
    fn = _decode_variant(mistake)
    assert any(_fails(p, fn) for p in DECODE_PINS), mistake


def test_correct_variant_passes_all_pins():
    fn = _decode_variant(None)
    assert not any(_fails(p, fn) for p in DECODE_PINS)


class _Eager(BlockAllocator):
    """Takes a new block as soon as the last one is full (ahead of need)."""

    def _reserve(self, seq_ids, n_new):
        slots, pairs = super()._reserve(seq_ids, n_new)
        for sid, n in zip(seq_ids, n_new):
            if n and self._ntok[sid] % self.block_size == 0:
                blk = self._pop()
                self._rc[blk] = 1
                self._table[sid].append(blk)
        return slots, pairs


class _FifoFree(BlockAllocator):
    """Pushes freed blocks in logical order (so the last one comes out first)."""

    def seq_free(self, seq_id):
        self._need(seq_id)
        for blk in self._table[seq_id]:
            self._rc[blk] -= 1
            if self._rc[blk] == 0:
                self._free.append(blk)
        del self._table[seq_id]
        del self._ntok[seq_id]


class _NoCow(BlockAllocator):
    """Writes into shared blocks in place."""

    def _reserve(self, seq_ids, n_new):
        bs = self.block_size
        slots = []
        for sid, n in zip(seq_ids, n_new):
            table = self._table[sid]
            for _ in range(n):
                pos = self._ntok[sid]
                lb, off = divmod(pos, bs)
                if off == 0:
                    blk = self._pop()
                    self._rc[blk] = 1
                    table.append(blk)
                slots.append(table[lb] * bs + off)
                self._ntok[sid] = pos + 1
        return slots, []


class _NoRollback(BlockAllocator):
    def seq_reserve(self, seq_ids, n_new, cow_cap=None):
        return self._reserve([int(s) for s in seq_ids], [int(n) for n in n_new])


def _alloc_pins(figures):
    return [lambda c: pins.check_seven_token_prompt(c),
            lambda c: pins.check_worked_batch(c, figures),
            lambda c: pins.check_free_lifo_reuse(c),
            lambda c: pins.check_fork_cow_trace(c),
            lambda c: pins.check_out_of_blocks_rollback(c, OutOfBlocks)]


@pytest.mark.parametrize("cls", [_Eager, _FifoFree, _NoCow, _NoRollback])
def test_allocator_mistake_is_caught(cls, page_figures):
    assert any(_fails(p, cls) for p in _alloc_pins(page_figures)), cls.__name__


def test_allocator_pins_pass_on_oracle(page_figures):
    assert not any(_fails(p, BlockAllocator) for p in _alloc_pins(page_figures))
