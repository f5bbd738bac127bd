"""Replays a workload's script through the oracle (CPU, test side only)."""

from __future__ import annotations

import numpy as np

from oracle import allocator as oa
from oracle import attention as oatt
from oracle import cache_ops as oc


class OracleCache:
    """Oracle allocator + NaN-poisoned pools, filled by a workload's script."""

    def __init__(self, w):
        self.w = w
        self.alloc = oa.BlockAllocator(w.num_blocks, w.block_size, w.free_order)
        self.k_cache = w.empty_pool()
        self.v_cache = w.empty_pool()
        self.log = []  # (op, result) for every script step

    def run(self, script=None):
        w = self.w
        for op in (w.script if script is None else script):
            if op[0] == "create":
                self.alloc.seq_create(op[1])
                self.log.append((op[0], None))
            elif op[0] == "fork":
                self.alloc.seq_fork(op[1], op[2])
                self.log.append((op[0], None))
            elif op[0] == "reserve":
                _, sids, ns, rows = op
                slots, pairs = self.alloc.seq_reserve(sids, ns)
                oc.copy_blocks(self.k_cache, self.v_cache, pairs)
                oc.cache_append(self.k_cache, self.v_cache, w.k_rows[rows], w.v_rows[rows],
                                slots, w.block_size)
                self.log.append((op[0], (np.array(slots, dtype=np.int64),
                                         np.array(pairs, dtype=np.int32).reshape(-1, 2))))
            else:
                raise ValueError(op[0])
        return self

    def tables(self, max_blocks=None):
        w = self.w
        if max_blocks is None:
            max_blocks = max(len(self.alloc.seq_block_table(s)) for s in w.seq_ids)
        rows, lens = self.alloc.block_tables(w.seq_ids, max_blocks)
        return np.array(rows, dtype=np.int32).reshape(len(w.seq_ids), max_blocks), \
            np.array(lens, dtype=np.int32)

    def decode(self, q=None, tables=None, lens=None):
        w = self.w
        if tables is None:
            tables, lens = self.tables()
        return oatt.paged_decode(w.q if q is None else q, self.k_cache, self.v_cache, tables,
                                 lens, w.block_size, w.scale, w.dtype)

    def contiguous(self):
        w = self.w
        ks = [w.k_rows[r] for r in w.logical_rows]
        vs = [w.v_rows[r] for r in w.logical_rows]
        return oatt.contiguous_decode(w.q, ks, vs, w.scale, w.dtype)
