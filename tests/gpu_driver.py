"""Replays a workload through the HIP library (test side; GPU)."""

from __future__ import annotations

import numpy as np
import torch

import paged_kv_cache_338_amd as pa


def to_torch(a, dtype, device):
    """Stored numpy values (float32, or bf16 / f16 as uint16 bits) -> device tensor."""
    if dtype in ("bf16", "f16"):
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
            torch.bfloat16 if dtype == "bf16" else torch.float16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


def to_numpy(t, dtype):
    t = t.detach().cpu().contiguous()
    if dtype in ("bf16", "f16"):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def widen_out(t, dtype):
    """GPU output -> float64 (exact)."""
    x = t.detach().cpu()
    return x.to(torch.float64).numpy() if dtype in ("bf16", "f16") else x.numpy().astype(np.float64)


class GpuCache:
    """C++ allocator + device pools filled by pa_copy_blocks / pa_cache_append."""

    def __init__(self, w, device="cuda:0", upload_rows=True):
        self.w = w
        self.device = device
        self.alloc = pa.Allocator(w.num_blocks, w.block_size, w.free_order)
        self.k_cache = to_torch(w.empty_pool(), w.dtype, device)
        self.v_cache = to_torch(w.empty_pool(), w.dtype, device)
        self.k_rows = to_torch(w.k_rows, w.dtype, device) if upload_rows else None
        self.v_rows = to_torch(w.v_rows, w.dtype, device) if upload_rows else None
        self.log = []

    def run(self, script=None, skip_rows=()):
        """Replays the script; bank rows in skip_rows are reserved but not
        appended (their slots are passed as -1)."""
        w = self.w
        skip = set(int(r) for r in skip_rows)
        for op in (w.script if script is None else script):
            if op[0] == "create":
                self.alloc.seq_create(op[1])
            elif op[0] == "fork":
                self.alloc.seq_fork(op[1], op[2])
            else:
                _, sids, ns, rows = op
                slots, pairs = self.alloc.seq_reserve(sids, ns, cow_cap=len(sids))
                if len(pairs):
                    pa.pa_copy_blocks(torch.from_numpy(np.ascontiguousarray(pairs)).to(self.device),
                                      self.k_cache, self.v_cache)
                idx = torch.from_numpy(np.asarray(rows, np.int64)).to(self.device)
                aslots = slots.copy()
                if skip:
                    aslots[[int(r) in skip for r in rows]] = -1
                pa.pa_cache_append(self.k_rows.index_select(0, idx).contiguous(),
                                   self.v_rows.index_select(0, idx).contiguous(),
                                   torch.from_numpy(aslots).to(self.device),
                                   self.k_cache, self.v_cache)
                self.log.append((slots.copy(), pairs.copy()))
        torch.cuda.synchronize()
        return self

    def tables(self, max_blocks=None):
        w = self.w
        if max_blocks is None:
            max_blocks = max(1, max(len(self.alloc.seq_block_table(s)) for s in w.seq_ids))
        t, l = self.alloc.build_block_tables(w.seq_ids, max_blocks)
        return t, l

    def decode(self, q=None, tables=None, lens=None, max_blocks=None):
        w = self.w
        if tables is None:
            tables, lens = self.tables(max_blocks)
        qd = to_torch(w.q if q is None else q, w.dtype, self.device)
        out = torch.empty_like(qd)
        pa.pa_decode(qd, self.k_cache, self.v_cache,
                     torch.from_numpy(np.ascontiguousarray(tables, np.int32)).to(self.device),
                     torch.from_numpy(np.ascontiguousarray(lens, np.int32)).to(self.device),
                     w.block_size, w.scale, out)
        torch.cuda.synchronize()
        return out
