// Host block allocator: free stack, per-block reference counts and one block
// table per sequence, with lazy allocation, fork and copy-on-write.
//
// Sources: "What is paged attention in vLLM, and why does it matter?"
// (interview.clozo.ai), Step 3 (table + free pool + per-block counts) and
// Step 4 (allocate only when the last block is full; blocks return to the
// pool on finish); "PagedAttention - AI Glossary" (modelrefs.com), How it
// works, items 2, 4 and 5 (grow block by block; shared prefixes by reference
// count; copy only the block being written).
//
// Preemption by swapping ("Paged Attention" glossary, Common questions, and
// the clozo.ai page, Follow-up questions, on running out of blocks: a
// preempted request's blocks move to CPU memory, or are dropped and
// recomputed): an optional pool of host blocks with its own LIFO stack;
// swap-out moves a whole sequence to host blocks in logical order and
// releases its device blocks as a free does (shared blocks stay with the
// other sharers); swap-in is the reverse, into private device blocks.  Both
// check the target pool first, so they change nothing when it is short.
//
// Automatic prefix caching (clozo.ai page, Trade-offs and edge cases, fourth
// point: full blocks are hashed, the least recently used are evicted): a
// full block's key is a chained 64-bit FNV-1a hash of its parent's key and
// its token ids, verified on a hit against the stored parent key and
// tokens.  Token ids come from pa_seq_match_prefix (normally the prompt);
// a block is cached when it becomes full during a reserve.  Released
// cached blocks wait on an LRU list; allocation takes free blocks first and
// then evicts the least recently used cached block.
//
// Every entry point gives the strong guarantee: pa_seq_reserve keeps an undo
// log while it walks the tokens and replays it backwards when it runs out of
// blocks or out of room for copy pairs, so a failed call leaves the free
// stack order, counts and tables exactly as they were.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <iterator>
#include <list>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pa_internal.h"

namespace {

// Key of one full block of registered tokens.
struct BlockKey {
  uint64_t key = 0;
  uint64_t parent = 0;
  std::vector<int32_t> tokens;
};

struct Sequence {
  std::vector<int32_t> table;  // logical block -> physical block (host block when swapped)
  int32_t num_tokens = 0;
  bool swapped = false;
  std::vector<BlockKey> keys;  // per full block of the registered tokens
};

// 64-bit FNV-1a (Fowler, Noll, Vo): per byte, xor then multiply.
constexpr uint64_t kFnvOffset = 0xCBF29CE484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001B3ull;

uint64_t fnv1a64(const uint8_t* p, size_t n, uint64_t h = kFnvOffset) {
  for (size_t i = 0; i < n; ++i) h = (h ^ p[i]) * kFnvPrime;
  return h;
}

// Parent key as 8 little-endian bytes, then each token as 4 (the x86-64 and
// gfx950 hosts are little-endian, so the in-memory bytes are those bytes).
uint64_t block_key(uint64_t parent, const int32_t* tokens, int32_t n) {
  uint8_t pb[8];
  std::memcpy(pb, &parent, 8);
  const uint64_t h = fnv1a64(pb, 8);
  return fnv1a64(reinterpret_cast<const uint8_t*>(tokens), sizeof(int32_t) * (size_t)n, h);
}

// One reversible change made by a reserve call.
struct Undo {
  enum Kind : uint8_t { kPop, kRefcount, kTableAppend, kTableSet, kTokens, kEvict,
                        kRegister } kind;
  Sequence* seq;
  int32_t a;  // block (kPop, kRefcount, kEvict, kRegister), logical index (kTableSet)
  int32_t b;  // old value (kRefcount, kTableSet, kTokens); saved key index (kRegister)
};

}  // namespace

struct pa_allocator {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> free_stack;  // top at back()
  std::vector<int32_t> refcount;
  std::unordered_map<int64_t, Sequence> seqs;
  std::vector<Undo> undo;  // reused between calls
  // Keys a kRegister overwrote, restored by the rollback: an evicted block
  // that the same call refills and registers under a new key must get its
  // old key back before the eviction itself is undone.
  std::vector<BlockKey> saved_keys;
  bool has_host = false;
  int32_t num_host_blocks = 0;
  std::vector<int32_t> host_free;  // top at back()
  // Prefix cache: per block whether it holds a key (and which), the key ->
  // block map, and the evictable (count 0) cached blocks, next evicted first.
  bool prefix_cache = false;
  std::vector<uint8_t> cached;
  std::vector<BlockKey> bkey;
  std::unordered_map<uint64_t, int32_t> block_of;
  std::list<int32_t> lru;
  std::vector<std::list<int32_t>::iterator> lru_pos;

  Sequence* find(int64_t id) {
    auto it = seqs.find(id);
    return it == seqs.end() ? nullptr : &it->second;
  }
  const Sequence* find(int64_t id) const {
    auto it = seqs.find(id);
    return it == seqs.end() ? nullptr : &it->second;
  }

  void rollback() {
    for (auto it = undo.rbegin(); it != undo.rend(); ++it) {
      switch (it->kind) {
        case Undo::kPop: free_stack.push_back(it->a); break;
        case Undo::kRefcount: refcount[it->a] = it->b; break;
        case Undo::kTableAppend: it->seq->table.pop_back(); break;
        case Undo::kTableSet: it->seq->table[it->a] = it->b; break;
        case Undo::kTokens: it->seq->num_tokens = it->b; break;
        case Undo::kEvict:
          cached[it->a] = 1;
          block_of[bkey[it->a].key] = it->a;
          lru.push_front(it->a);
          lru_pos[it->a] = lru.begin();
          break;
        case Undo::kRegister:
          cached[it->a] = 0;
          block_of.erase(bkey[it->a].key);
          bkey[it->a] = std::move(saved_keys[it->b]);
          break;
      }
    }
    undo.clear();
    saved_keys.clear();
  }

  bool pop(int32_t* blk) {
    if (!free_stack.empty()) {
      *blk = free_stack.back();
      free_stack.pop_back();
      undo.push_back({Undo::kPop, nullptr, *blk, 0});
      return true;
    }
    if (prefix_cache && !lru.empty()) {  // evict the least recently used cached block
      *blk = lru.front();
      lru.pop_front();
      cached[*blk] = 0;
      block_of.erase(bkey[*blk].key);
      undo.push_back({Undo::kEvict, nullptr, *blk, 0});
      return true;
    }
    return false;
  }

  int64_t available() const {
    return static_cast<int64_t>(free_stack.size()) + (prefix_cache ? lru.size() : 0);
  }

  // One reference fewer; at zero a cached block waits on the LRU list.
  void release(int32_t blk) {
    if (--refcount[blk] != 0) return;
    if (prefix_cache && cached[blk]) {
      lru.push_back(blk);
      lru_pos[blk] = std::prev(lru.end());
    } else {
      free_stack.push_back(blk);
    }
  }

  // Block lb of s just became full: cache it under its key if it has one
  // and the key is not held by another block.
  void maybe_register(Sequence* s, int32_t lb) {
    if (!prefix_cache || lb >= static_cast<int32_t>(s->keys.size())) return;
    const BlockKey& k = s->keys[lb];
    if (block_of.count(k.key)) return;
    const int32_t blk = s->table[lb];
    undo.push_back({Undo::kRegister, nullptr, blk, static_cast<int32_t>(saved_keys.size())});
    saved_keys.push_back(std::move(bkey[blk]));
    bkey[blk] = k;
    cached[blk] = 1;
    block_of[k.key] = blk;
  }

  void set_refcount(int32_t blk, int32_t value) {
    undo.push_back({Undo::kRefcount, nullptr, blk, refcount[blk]});
    refcount[blk] = value;
  }
};

extern "C" {

pa_status pa_allocator_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                              pa_allocator** out) {
  if (!out) return pa::fail(PA_ERR_INVALID_ARGUMENT, "out is NULL");
  *out = nullptr;
  if (num_blocks < 1 || block_size < 1)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "num_blocks (%d) and block_size (%d) must be >= 1",
                    num_blocks, block_size);
  pa_allocator* a = new (std::nothrow) pa_allocator;
  if (!a) return pa::fail(PA_ERR_INVALID_ARGUMENT, "host allocation failed");
  a->num_blocks = num_blocks;
  a->block_size = block_size;
  a->refcount.assign(num_blocks, 0);
  a->free_stack.resize(num_blocks);
  if (free_order) {
    std::vector<uint8_t> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t x = free_order[i];
      if (x < 0 || x >= num_blocks || seen[x]) {
        delete a;
        return pa::fail(PA_ERR_INVALID_ARGUMENT,
                        "free_order is not a permutation of 0..%d (entry %d = %d)",
                        num_blocks - 1, i, x);
      }
      seen[x] = 1;
    }
  }
  // The first block handed out is free_order[0]: it goes on top of the stack.
  for (int32_t i = 0; i < num_blocks; ++i)
    a->free_stack[num_blocks - 1 - i] = free_order ? free_order[i] : i;
  *out = a;
  return PA_OK;
}

void pa_allocator_destroy(pa_allocator* alloc) { delete alloc; }

pa_status pa_seq_create(pa_allocator* alloc, int64_t seq_id) {
  if (!alloc) return pa::fail(PA_ERR_INVALID_ARGUMENT, "allocator is NULL");
  if (alloc->find(seq_id))
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "sequence %lld exists", (long long)seq_id);
  alloc->seqs.emplace(seq_id, Sequence{});
  return PA_OK;
}

pa_status pa_seq_fork(pa_allocator* alloc, int64_t parent, int64_t child) {
  if (!alloc) return pa::fail(PA_ERR_INVALID_ARGUMENT, "allocator is NULL");
  const Sequence* p = alloc->find(parent);
  if (!p) return pa::fail(PA_ERR_UNKNOWN_SEQ, "unknown parent sequence %lld", (long long)parent);
  if (p->swapped)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "sequence %lld is swapped out", (long long)parent);
  if (alloc->find(child))
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "child sequence %lld exists", (long long)child);
  Sequence copy = *p;  // copy before emplace: emplace may rehash
  for (int32_t blk : copy.table) alloc->refcount[blk] += 1;
  alloc->seqs.emplace(child, std::move(copy));
  return PA_OK;
}

pa_status pa_seq_free(pa_allocator* alloc, int64_t seq_id) {
  if (!alloc) return pa::fail(PA_ERR_INVALID_ARGUMENT, "allocator is NULL");
  auto it = alloc->seqs.find(seq_id);
  if (it == alloc->seqs.end())
    return pa::fail(PA_ERR_UNKNOWN_SEQ, "unknown sequence %lld", (long long)seq_id);
  const std::vector<int32_t>& t = it->second.table;
  if (it->second.swapped) {
    for (auto r = t.rbegin(); r != t.rend(); ++r) alloc->host_free.push_back(*r);
  } else {
    for (auto r = t.rbegin(); r != t.rend(); ++r) alloc->release(*r);
  }
  alloc->seqs.erase(it);
  return PA_OK;
}

pa_status pa_seq_reserve(pa_allocator* alloc, const int64_t* seq_ids, const int32_t* n_new,
                         int32_t n, int64_t* slot_mapping_out, int32_t* cow_pairs_out,
                         int32_t cow_cap, int32_t* num_cow_out) {
  if (!alloc) return pa::fail(PA_ERR_INVALID_ARGUMENT, "allocator is NULL");
  if (n < 0) return pa::fail(PA_ERR_INVALID_ARGUMENT, "n = %d < 0", n);
  if (n > 0 && (!seq_ids || !n_new))
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "seq_ids / n_new is NULL");
  if (cow_cap < 0) return pa::fail(PA_ERR_INVALID_ARGUMENT, "cow_cap < 0");
  if (cow_cap > 0 && !cow_pairs_out)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "cow_pairs_out is NULL with cow_cap > 0");

  std::vector<Sequence*> seqs(n);
  std::unordered_set<int64_t> seen;
  seen.reserve(static_cast<size_t>(n) * 2);
  int64_t total = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (n_new[i] < 0)
      return pa::fail(PA_ERR_INVALID_ARGUMENT, "n_new[%d] = %d < 0", i, n_new[i]);
    seqs[i] = alloc->find(seq_ids[i]);
    if (!seqs[i])
      return pa::fail(PA_ERR_UNKNOWN_SEQ, "unknown sequence %lld", (long long)seq_ids[i]);
    if (seqs[i]->swapped)
      return pa::fail(PA_ERR_INVALID_ARGUMENT, "sequence %lld is swapped out",
                      (long long)seq_ids[i]);
    if (!seen.insert(seq_ids[i]).second)
      return pa::fail(PA_ERR_INVALID_ARGUMENT, "sequence %lld listed twice",
                      (long long)seq_ids[i]);
    if (static_cast<int64_t>(seqs[i]->num_tokens) + n_new[i] > INT32_MAX)
      return pa::fail(PA_ERR_INVALID_ARGUMENT, "sequence %lld would exceed INT32_MAX tokens",
                      (long long)seq_ids[i]);
    total += n_new[i];
  }
  if (total > 0 && !slot_mapping_out)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "slot_mapping_out is NULL");

  const int32_t bs = alloc->block_size;
  alloc->undo.clear();
  alloc->saved_keys.clear();
  int32_t pairs = 0;
  int64_t t = 0;
  for (int32_t i = 0; i < n; ++i) {
    Sequence* s = seqs[i];
    if (n_new[i] == 0) continue;
    alloc->undo.push_back({Undo::kTokens, s, 0, s->num_tokens});
    for (int32_t j = 0; j < n_new[i]; ++j) {
      const int32_t pos = s->num_tokens;
      const int32_t lb = pos / bs, off = pos % bs;
      if (off == 0) {
        int32_t blk;
        if (!alloc->pop(&blk)) {
          alloc->rollback();
          return pa::fail(PA_ERR_OUT_OF_BLOCKS, "no free block (pool of %d)", alloc->num_blocks);
        }
        alloc->set_refcount(blk, 1);
        s->table.push_back(blk);
        alloc->undo.push_back({Undo::kTableAppend, s, 0, 0});
      } else if (alloc->refcount[s->table[lb]] > 1) {
        const int32_t src = s->table[lb];
        int32_t dst;
        if (!alloc->pop(&dst)) {
          alloc->rollback();
          return pa::fail(PA_ERR_OUT_OF_BLOCKS, "no free block (pool of %d)", alloc->num_blocks);
        }
        alloc->set_refcount(src, alloc->refcount[src] - 1);
        alloc->set_refcount(dst, 1);
        alloc->undo.push_back({Undo::kTableSet, s, lb, src});
        s->table[lb] = dst;
        if (pairs < cow_cap) {
          cow_pairs_out[2 * pairs] = src;
          cow_pairs_out[2 * pairs + 1] = dst;
        }
        ++pairs;
      }
      slot_mapping_out[t++] = static_cast<int64_t>(s->table[lb]) * bs + off;
      s->num_tokens = pos + 1;
      if (off == bs - 1) alloc->maybe_register(s, lb);
    }
  }
  if (pairs > cow_cap) {
    // Checked after the walk so that running out of blocks is reported first.
    alloc->rollback();
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "%d copy pairs > cow_cap = %d", pairs, cow_cap);
  }
  alloc->undo.clear();
  alloc->saved_keys.clear();
  if (num_cow_out) *num_cow_out = pairs;
  return PA_OK;
}

pa_status pa_build_block_tables(const pa_allocator* alloc, const int64_t* seq_ids, int32_t n,
                                int32_t max_blocks_per_seq, int32_t* tables_out,
                                int32_t* context_lens_out) {
  if (!alloc) return pa::fail(PA_ERR_INVALID_ARGUMENT, "allocator is NULL");
  if (n < 0 || max_blocks_per_seq < 1)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "n = %d, max_blocks_per_seq = %d", n,
                    max_blocks_per_seq);
  if (n > 0 && (!seq_ids || !tables_out || !context_lens_out))
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "NULL array");
  for (int32_t i = 0; i < n; ++i) {
    const Sequence* s = alloc->find(seq_ids[i]);
    if (!s) return pa::fail(PA_ERR_UNKNOWN_SEQ, "unknown sequence %lld", (long long)seq_ids[i]);
    if (s->swapped)
      return pa::fail(PA_ERR_INVALID_ARGUMENT, "sequence %lld is swapped out",
                      (long long)seq_ids[i]);
    if (static_cast<int64_t>(s->table.size()) > max_blocks_per_seq)
      return pa::fail(PA_ERR_INVALID_ARGUMENT, "sequence %lld holds %zu blocks > %d",
                      (long long)seq_ids[i], s->table.size(), max_blocks_per_seq);
  }
  for (int32_t i = 0; i < n; ++i) {
    const Sequence* s = alloc->find(seq_ids[i]);
    int32_t* row = tables_out + static_cast<int64_t>(i) * max_blocks_per_seq;
    std::copy(s->table.begin(), s->table.end(), row);
    std::fill(row + s->table.size(), row + max_blocks_per_seq, -1);
    context_lens_out[i] = s->num_tokens;
  }
  return PA_OK;
}

pa_status pa_allocator_add_host_pool(pa_allocator* alloc, int32_t num_host_blocks,
                                     const int32_t* free_order) {
  if (!alloc) return pa::fail(PA_ERR_INVALID_ARGUMENT, "allocator is NULL");
  if (alloc->has_host) return pa::fail(PA_ERR_INVALID_ARGUMENT, "host pool exists");
  if (num_host_blocks < 1)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "num_host_blocks (%d) must be >= 1", num_host_blocks);
  if (free_order) {
    std::vector<uint8_t> seen(num_host_blocks, 0);
    for (int32_t i = 0; i < num_host_blocks; ++i) {
      const int32_t x = free_order[i];
      if (x < 0 || x >= num_host_blocks || seen[x])
        return pa::fail(PA_ERR_INVALID_ARGUMENT,
                        "free_order is not a permutation of 0..%d (entry %d = %d)",
                        num_host_blocks - 1, i, x);
      seen[x] = 1;
    }
  }
  alloc->host_free.resize(num_host_blocks);
  for (int32_t i = 0; i < num_host_blocks; ++i)
    alloc->host_free[num_host_blocks - 1 - i] = free_order ? free_order[i] : i;
  alloc->num_host_blocks = num_host_blocks;
  alloc->has_host = true;
  return PA_OK;
}

pa_status pa_seq_swap_out(pa_allocator* alloc, int64_t seq_id, int32_t* pairs_out, int32_t cap,
                          int32_t* num_pairs_out) {
  if (!alloc) return pa::fail(PA_ERR_INVALID_ARGUMENT, "allocator is NULL");
  Sequence* s = alloc->find(seq_id);
  if (!s) return pa::fail(PA_ERR_UNKNOWN_SEQ, "unknown sequence %lld", (long long)seq_id);
  if (s->swapped)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "sequence %lld is swapped out", (long long)seq_id);
  if (!alloc->has_host) return pa::fail(PA_ERR_INVALID_ARGUMENT, "no host pool");
  const int32_t n = static_cast<int32_t>(s->table.size());
  if (n > static_cast<int32_t>(alloc->host_free.size()))
    return pa::fail(PA_ERR_OUT_OF_BLOCKS, "no free host block (%zu free, %d needed)",
                    alloc->host_free.size(), n);
  if (cap < n) return pa::fail(PA_ERR_INVALID_ARGUMENT, "cap %d < %d pairs", cap, n);
  if (n > 0 && !pairs_out) return pa::fail(PA_ERR_INVALID_ARGUMENT, "pairs_out is NULL");
  for (int32_t i = 0; i < n; ++i) {
    const int32_t h = alloc->host_free.back();
    alloc->host_free.pop_back();
    pairs_out[2 * i] = s->table[i];
    pairs_out[2 * i + 1] = h;
  }
  for (int32_t i = n - 1; i >= 0; --i) alloc->release(s->table[i]);
  for (int32_t i = 0; i < n; ++i) s->table[i] = pairs_out[2 * i + 1];
  s->swapped = true;
  if (num_pairs_out) *num_pairs_out = n;
  return PA_OK;
}

pa_status pa_seq_swap_in(pa_allocator* alloc, int64_t seq_id, int32_t* pairs_out, int32_t cap,
                         int32_t* num_pairs_out) {
  if (!alloc) return pa::fail(PA_ERR_INVALID_ARGUMENT, "allocator is NULL");
  Sequence* s = alloc->find(seq_id);
  if (!s) return pa::fail(PA_ERR_UNKNOWN_SEQ, "unknown sequence %lld", (long long)seq_id);
  if (!s->swapped)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "sequence %lld is not swapped out",
                    (long long)seq_id);
  const int32_t n = static_cast<int32_t>(s->table.size());
  if (n > alloc->available())
    return pa::fail(PA_ERR_OUT_OF_BLOCKS, "no free block (%lld free, %d needed)",
                    (long long)alloc->available(), n);
  if (cap < n) return pa::fail(PA_ERR_INVALID_ARGUMENT, "cap %d < %d pairs", cap, n);
  if (n > 0 && !pairs_out) return pa::fail(PA_ERR_INVALID_ARGUMENT, "pairs_out is NULL");
  for (int32_t i = 0; i < n; ++i) {
    int32_t d = 0;
    alloc->pop(&d);  // cannot fail: checked above
    alloc->refcount[d] = 1;
    pairs_out[2 * i] = s->table[i];
    pairs_out[2 * i + 1] = d;
  }
  alloc->undo.clear();
  for (int32_t i = n - 1; i >= 0; --i) alloc->host_free.push_back(s->table[i]);
  for (int32_t i = 0; i < n; ++i) s->table[i] = pairs_out[2 * i + 1];
  s->swapped = false;
  if (num_pairs_out) *num_pairs_out = n;
  return PA_OK;
}

pa_status pa_allocator_enable_prefix_cache(pa_allocator* alloc) {
  if (!alloc) return pa::fail(PA_ERR_INVALID_ARGUMENT, "allocator is NULL");
  if (!alloc->prefix_cache) {
    alloc->prefix_cache = true;
    alloc->cached.assign(alloc->num_blocks, 0);
    alloc->bkey.assign(alloc->num_blocks, BlockKey{});
    alloc->lru_pos.assign(alloc->num_blocks, alloc->lru.end());
  }
  return PA_OK;
}

pa_status pa_seq_match_prefix(pa_allocator* alloc, int64_t seq_id, const int32_t* tokens,
                              int32_t n, int32_t* num_cached_out) {
  if (!alloc) return pa::fail(PA_ERR_INVALID_ARGUMENT, "allocator is NULL");
  Sequence* s = alloc->find(seq_id);
  if (!s) return pa::fail(PA_ERR_UNKNOWN_SEQ, "unknown sequence %lld", (long long)seq_id);
  if (!alloc->prefix_cache) return pa::fail(PA_ERR_INVALID_ARGUMENT, "prefix cache is off");
  if (s->swapped || !s->table.empty() || s->num_tokens != 0)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "sequence %lld is not empty", (long long)seq_id);
  if (n < 0 || (n > 0 && !tokens))
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "n = %d / tokens is NULL", n);
  const int32_t bs = alloc->block_size;
  const int32_t nfull = n / bs;
  std::vector<BlockKey> keys(nfull);
  uint64_t parent = 0;
  for (int32_t i = 0; i < nfull; ++i) {
    keys[i].parent = parent;
    keys[i].tokens.assign(tokens + (int64_t)i * bs, tokens + (int64_t)(i + 1) * bs);
    keys[i].key = block_key(parent, tokens + (int64_t)i * bs, bs);
    parent = keys[i].key;
  }
  const int32_t max_hits = n > 0 ? (n - 1) / bs : 0;
  int32_t hits = 0;
  for (; hits < max_hits; ++hits) {
    const BlockKey& k = keys[hits];
    auto it = alloc->block_of.find(k.key);
    if (it == alloc->block_of.end()) break;
    const int32_t blk = it->second;
    const BlockKey& have = alloc->bkey[blk];
    if (have.parent != k.parent || have.tokens != k.tokens) break;
    if (alloc->refcount[blk] == 0) alloc->lru.erase(alloc->lru_pos[blk]);
    alloc->refcount[blk] += 1;
    s->table.push_back(blk);
  }
  s->keys = std::move(keys);
  s->num_tokens = hits * bs;
  if (num_cached_out) *num_cached_out = hits * bs;
  return PA_OK;
}

int32_t pa_allocator_num_cached(const pa_allocator* alloc) {
  return alloc ? static_cast<int32_t>(alloc->lru.size()) : -1;
}

pa_status pa_allocator_cached_list(const pa_allocator* alloc, int32_t* out, int32_t cap,
                                   int32_t* len) {
  if (!alloc || !len) return pa::fail(PA_ERR_INVALID_ARGUMENT, "NULL argument");
  const int32_t nc = static_cast<int32_t>(alloc->lru.size());
  *len = nc;
  if (cap < nc) return pa::fail(PA_ERR_INVALID_ARGUMENT, "cap %d < %d cached blocks", cap, nc);
  if (nc > 0 && !out) return pa::fail(PA_ERR_INVALID_ARGUMENT, "out is NULL");
  std::copy(alloc->lru.begin(), alloc->lru.end(), out);
  return PA_OK;
}

pa_status pa_block_prefix_key(const pa_allocator* alloc, int32_t block, int32_t* cached_out,
                              uint64_t* key_out) {
  if (!alloc || !cached_out || !key_out)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "NULL argument");
  if (block < 0 || block >= alloc->num_blocks)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "block %d outside [0, %d)", block, alloc->num_blocks);
  const bool c = alloc->prefix_cache && alloc->cached[block];
  *cached_out = c ? 1 : 0;
  *key_out = c ? alloc->bkey[block].key : 0;
  return PA_OK;
}

pa_status pa_seq_is_swapped(const pa_allocator* alloc, int64_t seq_id, int32_t* out) {
  if (!alloc || !out) return pa::fail(PA_ERR_INVALID_ARGUMENT, "NULL argument");
  const Sequence* s = alloc->find(seq_id);
  if (!s) return pa::fail(PA_ERR_UNKNOWN_SEQ, "unknown sequence %lld", (long long)seq_id);
  *out = s->swapped ? 1 : 0;
  return PA_OK;
}

int32_t pa_allocator_num_free_host(const pa_allocator* alloc) {
  return alloc && alloc->has_host ? static_cast<int32_t>(alloc->host_free.size()) : -1;
}

pa_status pa_allocator_host_free_list(const pa_allocator* alloc, int32_t* out, int32_t cap,
                                      int32_t* len) {
  if (!alloc || !len) return pa::fail(PA_ERR_INVALID_ARGUMENT, "NULL argument");
  if (!alloc->has_host) return pa::fail(PA_ERR_INVALID_ARGUMENT, "no host pool");
  const int32_t nf = static_cast<int32_t>(alloc->host_free.size());
  *len = nf;
  if (cap < nf) return pa::fail(PA_ERR_INVALID_ARGUMENT, "cap %d < %d free blocks", cap, nf);
  if (nf > 0 && !out) return pa::fail(PA_ERR_INVALID_ARGUMENT, "out is NULL");
  std::copy(alloc->host_free.rbegin(), alloc->host_free.rend(), out);
  return PA_OK;
}

int32_t pa_allocator_num_free(const pa_allocator* alloc) {
  return alloc ? static_cast<int32_t>(alloc->free_stack.size()) : -1;
}

pa_status pa_allocator_free_list(const pa_allocator* alloc, int32_t* out, int32_t cap,
                                 int32_t* len) {
  if (!alloc || !len) return pa::fail(PA_ERR_INVALID_ARGUMENT, "NULL argument");
  const int32_t nf = static_cast<int32_t>(alloc->free_stack.size());
  *len = nf;
  if (cap < nf) return pa::fail(PA_ERR_INVALID_ARGUMENT, "cap %d < %d free blocks", cap, nf);
  if (nf > 0 && !out) return pa::fail(PA_ERR_INVALID_ARGUMENT, "out is NULL");
  std::copy(alloc->free_stack.rbegin(), alloc->free_stack.rend(), out);
  return PA_OK;
}

pa_status pa_block_refcount(const pa_allocator* alloc, int32_t block, int32_t* out) {
  if (!alloc || !out) return pa::fail(PA_ERR_INVALID_ARGUMENT, "NULL argument");
  if (block < 0 || block >= alloc->num_blocks)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "block %d outside 0..%d", block,
                    alloc->num_blocks - 1);
  *out = alloc->refcount[block];
  return PA_OK;
}

pa_status pa_seq_block_table(const pa_allocator* alloc, int64_t seq_id, int32_t* out, int32_t cap,
                             int32_t* len) {
  if (!alloc || !len) return pa::fail(PA_ERR_INVALID_ARGUMENT, "NULL argument");
  const Sequence* s = alloc->find(seq_id);
  if (!s) return pa::fail(PA_ERR_UNKNOWN_SEQ, "unknown sequence %lld", (long long)seq_id);
  const int32_t nb = static_cast<int32_t>(s->table.size());
  *len = nb;
  if (cap < nb) return pa::fail(PA_ERR_INVALID_ARGUMENT, "cap %d < %d blocks", cap, nb);
  if (nb > 0 && !out) return pa::fail(PA_ERR_INVALID_ARGUMENT, "out is NULL");
  std::copy(s->table.begin(), s->table.end(), out);
  return PA_OK;
}

pa_status pa_seq_num_tokens(const pa_allocator* alloc, int64_t seq_id, int32_t* out) {
  if (!alloc || !out) return pa::fail(PA_ERR_INVALID_ARGUMENT, "NULL argument");
  const Sequence* s = alloc->find(seq_id);
  if (!s) return pa::fail(PA_ERR_UNKNOWN_SEQ, "unknown sequence %lld", (long long)seq_id);
  *out = s->num_tokens;
  return PA_OK;
}

}  // extern "C"
