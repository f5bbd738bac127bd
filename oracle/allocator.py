"""Oracle block allocator (plain Python; test infrastructure only).

What it models
--------------
* A pool of ``num_blocks`` physical KV blocks of ``block_size`` token slots
  each, owned by the runtime, any of which can hold any logical block
  [P1 "Paged Attention", body: the runtime owns a pool of physical blocks;
  P3 "What is paged attention in vLLM...", Step 2: a free block fits any
  request].
* A free list and a reference count per block, kept beside the per-sequence
  block tables [P3, Step 3: the block manager keeps the table next to a pool
  of free blocks and one reference count per block].
* A block table per sequence: logical block index (token order) -> physical
  block id.  Token position ``pos`` lives in logical block ``pos // bs`` at
  offset ``pos % bs`` [P1, body: the kernel derives logical block and offset
  and looks up the physical id].  The filled-slot count of each table entry
  is not stored; it follows from the sequence's token count.
* Lazy allocation: a block is taken only when a token arrives and the last
  block is full, never for a reserved maximum [P3, Step 4; P2 "PagedAttention
  — AI Glossary", How it works, item 2].
* Free on finish: every block whose count drops to zero returns to the free
  pool and can be taken by the next request at once [P3, Step 4].
* Prefix sharing by reference count: a fork points the child's table at the
  parent's physical blocks and raises their counts [P2, How it works,
  item 4; P3, Trade-offs and edge cases, third point].
* Copy-on-write: when a sequence is about to write into a block that other
  sequences still point at, only that block is duplicated; the writer's
  table is redirected to the copy and the (source, destination) pair is
  reported so the caller can copy the bytes [P2, How it works, item 5;
  P3, Trade-offs, third point].

Readings adopted where the pages are silent (stated once, used everywhere):

* The free list is a LIFO stack.  ``free_order`` (a permutation of the block
  ids, default ascending) is the order in which a fresh allocator hands
  blocks out.  Freeing pushes a sequence's blocks in reverse logical order,
  so its logical block 0 is handed out first afterwards.
* Copy-on-write fires iff the block about to be written is a partially
  filled tail whose count is above one.  Sequences are processed in call
  order, so the last remaining sharer writes in place.
* A slot is ``physical_block * block_size + offset``.
* A call that runs out of blocks changes nothing (all-or-nothing over the
  whole call) and raises ``OutOfBlocks``; the policy for that case belongs
  to the caller [P1, FAQ "What happens when the GPU runs out of KV blocks?"].

Preemption by swapping [P1, Common questions, "What happens when the GPU runs
out of KV blocks?": the runtime may move blocks to CPU memory, or drop them
and recompute from the tokens; P3, Follow-up questions, "What happens when
the GPU runs out of free blocks?": a preempted request's blocks are swapped to
CPU memory or dropped and recomputed later in one prefill pass].  Readings:

* An optional second pool of host (CPU memory) blocks with its own LIFO free
  stack (``add_host_pool``), handed out in ``free_order`` like the device
  pool.
* ``swap_out`` moves a whole sequence: one host block per logical block, in
  logical order, with a (device block, host block) pair per block for the
  caller's copy; then the device blocks are released exactly as by a free
  (reverse logical order, pushed when their count reaches zero).  A block
  the sequence shares with others is copied and stays on the device for
  them.
* ``swap_in`` is the reverse: one fresh device block per logical block (count
  1), a (host block, device block) pair each, then the host blocks return to
  the host stack in reverse logical order.  Sharing is not restored.
* Both are all-or-nothing (``OutOfBlocks`` when the target pool is short).
  A swapped-out sequence cannot reserve, fork or build a table; freeing it
  returns its host blocks.  The drop-and-recompute path needs no new state:
  free the sequence, create it again, reserve its tokens and prefill.

Automatic prefix caching [P3, Trade-offs and edge cases, fourth point: full
blocks are hashed and the least recently used are evicted; P1, Common
questions: a runtime short of blocks may evict cached prefixes].  Readings:

* A full block's key is a chained 64-bit FNV-1a hash: of the parent block's
  key (0 for block 0) as 8 little-endian bytes, then the block's token ids
  as 4-byte little-endian integers.  A hit also compares the stored parent
  key and token ids, so a hash collision cannot alias two prefixes.
* Keys come from token ids the caller registers for an empty sequence
  (``match_prefix``, normally the prompt); blocks of tokens it never
  registered (generated tokens) are not cached.  A block is entered in the
  cache when it becomes full during a reserve; the first block to hold a
  key keeps it.
* ``match_prefix`` takes the longest run of cached blocks from block 0, at
  most ``(n - 1) // bs`` of them so that at least one token is computed,
  and sets the sequence's length to the tokens they hold.
* A cached block whose count drops to zero is not freed but queued as
  evictable, most recently released last; a hit takes it back.  Blocks are
  taken from the free stack first, and only when it is empty is the least
  recently used cached block evicted (its key dropped).
"""

from __future__ import annotations

import copy


class AllocatorError(Exception):
    """Base class; ``status`` names the C-ABI status the condition maps to."""

    status = "ERROR"


class InvalidArgument(AllocatorError):
    status = "INVALID_ARGUMENT"


class OutOfBlocks(AllocatorError):
    status = "OUT_OF_BLOCKS"


class UnknownSeq(AllocatorError):
    status = "UNKNOWN_SEQ"


class BlockAllocator:
    """Free stack + reference counts + per-sequence tables."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        if num_blocks < 1 or block_size < 1:
            raise InvalidArgument("num_blocks and block_size must be >= 1")
        order = list(range(num_blocks)) if free_order is None else [int(x) for x in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise InvalidArgument("free_order must be a permutation of 0..num_blocks-1")
        self.num_blocks = num_blocks
        self.block_size = block_size
        # Stack with its top at the end: the first block handed out is order[0].
        self._free = list(reversed(order))
        self._rc = [0] * num_blocks
        self._table: dict[int, list[int]] = {}
        self._ntok: dict[int, int] = {}
        self._host_free: list[int] | None = None  # host stack, top at the end
        self._swapped: set[int] = set()
        self._pc = False                   # prefix caching on
        self._block_of: dict[int, int] = {}    # key -> cached block
        self._key_of: dict[int, tuple] = {}    # cached block -> (key, parent key, tokens)
        self._lru: list[int] = []          # evictable cached blocks, next evicted first
        self._keys: dict[int, list] = {}   # seq -> [(key, parent key, tokens)] per full block

    # ------------------------------------------------------------------ state
    def num_free(self) -> int:
        return len(self._free)

    def free_list(self) -> list[int]:
        """Free blocks, the one handed out next first."""
        return list(reversed(self._free))

    def refcount(self, block: int) -> int:
        if not 0 <= block < self.num_blocks:
            raise InvalidArgument("block id out of range")
        return self._rc[block]

    def seq_block_table(self, seq_id: int) -> list[int]:
        self._need(seq_id)
        return list(self._table[seq_id])

    def seq_num_tokens(self, seq_id: int) -> int:
        self._need(seq_id)
        return self._ntok[seq_id]

    def seq_ids(self) -> list[int]:
        return sorted(self._table)

    def num_cached(self) -> int:
        return len(self._lru)

    def cached_list(self) -> list[int]:
        """Evictable cached blocks, the one evicted next first."""
        return list(self._lru)

    def block_key(self, block: int):
        """The key of a cached block, or None."""
        k = self._key_of.get(block)
        return None if k is None else k[0]

    def num_free_host(self) -> int:
        return -1 if self._host_free is None else len(self._host_free)

    def host_free_list(self) -> list[int]:
        if self._host_free is None:
            raise InvalidArgument("no host pool")
        return list(reversed(self._host_free))

    def seq_is_swapped(self, seq_id: int) -> bool:
        self._need(seq_id)
        return seq_id in self._swapped

    # --------------------------------------------------------- prefix cache
    def enable_prefix_cache(self) -> None:
        self._pc = True

    def match_prefix(self, seq_id: int, tokens) -> int:
        """Registers the token ids of an empty sequence and takes the cached
        blocks of its longest cached prefix; returns the tokens they hold."""
        self._need(seq_id)
        if not self._pc:
            raise InvalidArgument("prefix cache is off")
        if seq_id in self._swapped or self._table[seq_id] or self._ntok[seq_id]:
            raise InvalidArgument("sequence is not empty")
        toks = [int(t) for t in tokens]
        bs = self.block_size
        keys, parent = [], 0
        for i in range(len(toks) // bs):
            blk_toks = tuple(toks[i * bs:(i + 1) * bs])
            key = block_key(parent, blk_toks)
            keys.append((key, parent, blk_toks))
            parent = key
        self._keys[seq_id] = keys
        hits = 0
        for key, parent, blk_toks in keys[:(len(toks) - 1) // bs if toks else 0]:
            blk = self._block_of.get(key)
            if blk is None or self._key_of[blk] != (key, parent, blk_toks):
                break
            if self._rc[blk] == 0:
                self._lru.remove(blk)
            self._rc[blk] += 1
            self._table[seq_id].append(blk)
            hits += 1
        self._ntok[seq_id] = hits * bs
        return hits * bs

    def _release(self, blk: int) -> None:
        """One reference fewer; at zero a cached block queues for eviction."""
        self._rc[blk] -= 1
        if self._rc[blk] == 0:
            if blk in self._key_of:
                self._lru.append(blk)
            else:
                self._free.append(blk)

    # ------------------------------------------------------------ host pool
    def add_host_pool(self, num_host_blocks: int, free_order=None) -> None:
        if self._host_free is not None:
            raise InvalidArgument("host pool exists")
        if num_host_blocks < 1:
            raise InvalidArgument("num_host_blocks must be >= 1")
        order = (list(range(num_host_blocks)) if free_order is None
                 else [int(x) for x in free_order])
        if sorted(order) != list(range(num_host_blocks)):
            raise InvalidArgument("free_order must be a permutation")
        self._host_free = list(reversed(order))

    def swap_out(self, seq_id: int):
        """Move the sequence to host blocks; returns (device, host) pairs."""
        self._need(seq_id)
        if seq_id in self._swapped:
            raise InvalidArgument("sequence is swapped out")
        if self._host_free is None:
            raise InvalidArgument("no host pool")
        table = self._table[seq_id]
        if len(table) > len(self._host_free):
            raise OutOfBlocks("no free host block")
        host = [self._host_free.pop() for _ in table]
        pairs = list(zip(table, host))
        for blk in reversed(table):
            self._release(blk)
        self._table[seq_id] = host
        self._swapped.add(seq_id)
        return pairs

    def swap_in(self, seq_id: int):
        """Move a swapped-out sequence back; returns (host, device) pairs."""
        self._need(seq_id)
        if seq_id not in self._swapped:
            raise InvalidArgument("sequence is not swapped out")
        host = self._table[seq_id]
        if len(host) > len(self._free) + len(self._lru):
            raise OutOfBlocks("no free block")
        dev = [self._pop() for _ in host]
        for blk in dev:
            self._rc[blk] = 1
        pairs = list(zip(host, dev))
        for blk in reversed(host):
            self._host_free.append(blk)
        self._table[seq_id] = dev
        self._swapped.discard(seq_id)
        return pairs

    # -------------------------------------------------------------- sequences
    def seq_create(self, seq_id: int) -> None:
        if seq_id in self._table:
            raise InvalidArgument("sequence exists")
        self._table[seq_id] = []
        self._ntok[seq_id] = 0

    def seq_fork(self, parent: int, child: int) -> None:
        """Child shares every physical block of the parent (count + 1 each)."""
        self._need(parent)
        if parent in self._swapped:
            raise InvalidArgument("sequence is swapped out")
        if child in self._table:
            raise InvalidArgument("child exists")
        self._table[child] = list(self._table[parent])
        self._ntok[child] = self._ntok[parent]
        if parent in self._keys:
            self._keys[child] = list(self._keys[parent])
        for blk in self._table[child]:
            self._rc[blk] += 1

    def seq_free(self, seq_id: int) -> None:
        """Drop one reference to each block; zero-count blocks rejoin the pool."""
        self._need(seq_id)
        if seq_id in self._swapped:
            self._host_free.extend(reversed(self._table[seq_id]))
            self._swapped.discard(seq_id)
        else:
            for blk in reversed(self._table[seq_id]):
                self._release(blk)
        del self._table[seq_id]
        del self._ntok[seq_id]
        self._keys.pop(seq_id, None)

    def seq_reserve(self, seq_ids, n_new, cow_cap=None):
        """Give ``n_new[i]`` new token slots to ``seq_ids[i]``, in call order.

        Returns ``(slot_mapping, cow_pairs)``: one slot per new token,
        sequence-major, and the (source, destination) block pairs whose
        bytes must be copied before the new tokens are written.
        """
        seq_ids = [int(s) for s in seq_ids]
        n_new = [int(n) for n in n_new]
        if len(seq_ids) != len(n_new):
            raise InvalidArgument("length mismatch")
        seen = set()
        for sid, n in zip(seq_ids, n_new):
            if n < 0:
                raise InvalidArgument("negative token count")
            if sid not in self._table:
                raise UnknownSeq(f"unknown sequence {sid}")
            if sid in self._swapped:
                raise InvalidArgument("sequence is swapped out")
            if sid in seen:
                raise InvalidArgument("sequence listed twice")
            seen.add(sid)

        saved = (list(self._free), list(self._rc),
                 copy.deepcopy(self._table), dict(self._ntok), list(self._lru),
                 dict(self._block_of), dict(self._key_of))
        try:
            slots, pairs = self._reserve(seq_ids, n_new)
            if cow_cap is not None and len(pairs) > cow_cap:
                raise InvalidArgument("copy-on-write pair capacity too small")
        except AllocatorError:
            (self._free, self._rc, self._table, self._ntok, self._lru, self._block_of,
             self._key_of) = saved
            raise
        return slots, pairs

    def block_tables(self, seq_ids, max_blocks: int):
        """Rows of physical ids padded with -1, plus each sequence's length."""
        rows, lens = [], []
        for sid in seq_ids:
            sid = int(sid)
            self._need(sid)
            if sid in self._swapped:
                raise InvalidArgument("sequence is swapped out")
            tab = self._table[sid]
            if len(tab) > max_blocks:
                raise InvalidArgument("table longer than max_blocks")
            rows.append(tab + [-1] * (max_blocks - len(tab)))
            lens.append(self._ntok[sid])
        return rows, lens

    # ---------------------------------------------------------------- private
    def _need(self, seq_id: int) -> None:
        if seq_id not in self._table:
            raise UnknownSeq(f"unknown sequence {seq_id}")

    def _pop(self) -> int:
        if self._free:
            return self._free.pop()
        if self._lru:  # evict the least recently used cached block
            blk = self._lru.pop(0)
            del self._block_of[self._key_of.pop(blk)[0]]
            return blk
        raise OutOfBlocks("no free block")

    def _reserve(self, seq_ids, n_new):
        bs = self.block_size
        slots, pairs = [], []
        for sid, n in zip(seq_ids, n_new):
            table = self._table[sid]
            for _ in range(n):
                pos = self._ntok[sid]
                lb, off = divmod(pos, bs)
                if off == 0:
                    # The last block is full (or there is none): take a block.
                    blk = self._pop()
                    self._rc[blk] = 1
                    table.append(blk)
                elif self._rc[table[lb]] > 1:
                    # Writing into a block others still read: copy it first.
                    src = table[lb]
                    dst = self._pop()
                    self._rc[src] -= 1
                    self._rc[dst] = 1
                    table[lb] = dst
                    pairs.append((src, dst))
                slots.append(table[lb] * bs + off)
                self._ntok[sid] = pos + 1
                keys = self._keys.get(sid)
                if off == bs - 1 and keys is not None and lb < len(keys):
                    key = keys[lb][0]
                    if key not in self._block_of:  # the block is full: cache it
                        self._block_of[key] = table[lb]
                        self._key_of[table[lb]] = keys[lb]
        return slots, pairs


FNV64_OFFSET = 0xCBF29CE484222325
FNV64_PRIME = 0x100000001B3


def fnv1a64(data: bytes, h: int = FNV64_OFFSET) -> int:
    """64-bit FNV-1a (Fowler, Noll, Vo): for each byte, xor then multiply."""
    for byte in data:
        h = ((h ^ byte) * FNV64_PRIME) & 0xFFFFFFFFFFFFFFFF
    return h


def block_key(parent: int, tokens) -> int:
    """Key of a full block: FNV-1a over the parent key (8 bytes LE) and the
    token ids (4 bytes LE each)."""
    data = int(parent).to_bytes(8, "little") + b"".join(
        int(t).to_bytes(4, "little", signed=True) for t in tokens)
    return fnv1a64(data)
