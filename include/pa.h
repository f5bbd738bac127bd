/*
 * pa.h - C ABI of the paged KV cache library (gfx950 / MI355X).
 *
 * The library implements the hot path of a paged KV cache for LLM decode:
 * K and V live in fixed-size blocks scattered through a physical pool, and a
 * per-sequence block table maps each logical token position to
 * (logical block, offset) and then to a physical block id.
 *
 * Sources (web pages; cited by title and section):
 *   [P1] "Paged Attention", klaylearn.com glossary
 *   [P2] "PagedAttention - AI Glossary", modelrefs.com
 *   [P3] "What is paged attention in vLLM, and why does it matter?",
 *        interview.clozo.ai blog
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every call returns a pa_status and never throws.  On an error the
 *   thread-local text from pa_last_error() says what was wrong.
 * - Device operations take DEVICE pointers owned by the caller (the library
 *   never allocates or frees device memory) and a hipStream_t passed as
 *   void*.  They only enqueue work on that stream and return; ordering
 *   between them (copy, then append, then decode) is the caller's stream
 *   order.  Host-checkable arguments are validated before anything is
 *   enqueued; a rejected call enqueues nothing.  Kernel launch failures come
 *   back as PA_ERR_DEVICE.
 * - Contents of device arrays (slots, table entries, lengths, pairs) are
 *   preconditions the host cannot check without a copy.  The kernels never
 *   touch memory outside the buffers described here: slots or block ids
 *   outside the pool are skipped (append, copy) or clamped into it (decode,
 *   whose output for such a sequence is then unspecified), and lengths are
 *   clamped to max_blocks_per_seq * block_size.
 * - Alignment: q, out, k, v, k_cache and v_cache 16 bytes; int64 arrays 8
 *   bytes; int32 arrays 4 bytes; the decode workspace 256 bytes.  A
 *   misaligned pointer is PA_ERR_INVALID_ARGUMENT.
 * - KV pool layout: two pools, k_cache and v_cache, each
 *   [num_blocks][num_kv_heads][block_size][head_dim], row-major, values of
 *   the pool's dtype.  One (block, KV head) tile is contiguous.
 * - Slot of a token: physical_block * block_size + offset_in_block, int64.
 * - Block tables: int32 [num_seqs][max_blocks_per_seq], row b lists the
 *   physical blocks of sequence b in logical (token) order; entries past
 *   ceil(context_len / block_size) are never read (pad with -1).
 * - Host allocator handles are not thread-safe; use one per thread or lock.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 1

typedef int32_t pa_status;
#define PA_OK 0
#define PA_ERR_INVALID_ARGUMENT 1
#define PA_ERR_OUT_OF_BLOCKS 2
#define PA_ERR_UNKNOWN_SEQ 3
#define PA_ERR_UNSUPPORTED 4
#define PA_ERR_DEVICE 5

typedef int32_t pa_dtype;
#define PA_F32 0
#define PA_BF16 1
#define PA_F16 2 /* IEEE binary16 */

/* Shape of one KV pool pair.  Supported: block_size a power of two in
 * [1, 256]; head_dim 64 or 128; dtype PA_F32, PA_BF16 or PA_F16.  The two
 * 16-bit formats halve every block against fp32 [P3 Trade-offs and edge
 * cases, fourth point: narrower cache values shrink every block; P3 Step 1:
 * 2-byte values]; attention computes in fp32 and rounds its probabilities
 * and output to the pool's format. */
typedef struct pa_cache_desc {
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  pa_dtype dtype;
} pa_cache_desc;

/* Version of this header the library was built from (PA_ABI_VERSION). */
int32_t pa_abi_version(void);

/* Static name of a status code ("PA_OK", ...); "PA_UNKNOWN_STATUS" else. */
const char* pa_status_string(pa_status status);

/* Detail of the last error raised on the calling thread ("" if none).  The
 * pointer stays valid until the thread's next library call. */
const char* pa_last_error(void);

/* PA_OK if the library has kernels for this pool shape and query-head count
 * (num_q_heads a multiple of num_kv_heads, group size num_q_heads /
 * num_kv_heads in [1, 16]); PA_ERR_UNSUPPORTED or PA_ERR_INVALID_ARGUMENT
 * otherwise. */
pa_status pa_supported(const pa_cache_desc* desc, int32_t num_q_heads);

/* Process-wide tuning knobs.  Each changes only how work is spread over
 * the GPU or how it uses the caches, never the result beyond fp32
 * summation order; 0 (the default) lets the library choose.  Read by every
 * later call of the operation (atomically; any thread may set them).
 *   PA_TUNE_DECODE_WORKGROUPS: workgroups of pa_decode's grid, in
 *     [1, 1024] (default 256, one per compute unit).
 *   PA_TUNE_PREFILL_KEY_TILES: key tiles of 32 keys per piece when
 *     pa_prefill_split splits (default: from the shape, at least 48).
 *   PA_TUNE_DECODE_KV_CACHED: 0 (default): pa_decode / pa_decode_append
 *     read K and V with non-temporal loads (each block is read once per
 *     call, so keeping it in the caches only evicts what the call reuses);
 *     1: ordinary cached loads, for batches whose sequences share blocks
 *     ("What is paged attention in vLLM, and why does it matter?",
 *     Trade-offs, fourth point: a shared prefix is read by every sharer in
 *     the same call and is then served from the caches).
 * INVALID_ARGUMENT for an unknown key or a value out of range. */
typedef int32_t pa_tuning_key;
#define PA_TUNE_DECODE_WORKGROUPS 1
#define PA_TUNE_PREFILL_KEY_TILES 2
#define PA_TUNE_DECODE_KV_CACHED 3
pa_status pa_set_tuning(pa_tuning_key key, int32_t value);
pa_status pa_get_tuning(pa_tuning_key key, int32_t* value);

/* ---------------------------------------------------------------- device */

/* Slot-mapped append [P3 Step 4: each decode step writes the new token's
 * keys and values into the last block; P1 body: prefill fills the blocks of
 * the prompt the same way].
 *
 * For every t < num_tokens with slot = slot_mapping[t] >= 0:
 *   k_cache[slot / bs][h][slot % bs][:] = k[t][h][:]   for every KV head h
 *   v_cache[...]                        = v[t][h][:]
 * k, v:          device, [num_tokens][num_kv_heads][head_dim], pool dtype.
 * slot_mapping:  device int64 [num_tokens]; negative = skip (padding);
 *                non-negative slots must be distinct within one call.
 * Exact bit copy.  num_tokens == 0 enqueues nothing. */
pa_status pa_cache_append(const void* k, const void* v, const int64_t* slot_mapping,
                          int32_t num_tokens, void* k_cache, void* v_cache,
                          const pa_cache_desc* desc, void* stream);

/* Whole-block copy for copy-on-write [P2 How it works, item 5: only the
 * block being written is copied; P3 Trade-offs, third point].
 *
 * For every pair i < num_pairs: block dst = src_dst_pairs[2i+1] of both pools
 * becomes a bit copy of block src = src_dst_pairs[2i] (all heads, all slots).
 * src_dst_pairs: device int32 [num_pairs][2].  Destinations must be
 * distinct and must not appear as sources.  num_pairs == 0 enqueues
 * nothing. */
pa_status pa_copy_blocks(const int32_t* src_dst_pairs, int32_t num_pairs, void* k_cache,
                         void* v_cache, const pa_cache_desc* desc, void* stream);

/* Whole-block moves between two pool pairs of one geometry, for preemption
 * by swapping [P1 Common questions, "What happens when the GPU runs out of
 * KV blocks?": blocks may move to CPU memory; P3 Follow-up questions, "What
 * happens when the GPU runs out of free blocks?": a preempted request's
 * blocks are swapped to CPU memory, or dropped and recomputed].
 *
 * For every pair i < num_pairs: block dst = src_dst_pairs[2i+1] of dst_k and
 * dst_v becomes a bit copy of block src = src_dst_pairs[2i] of src_k and
 * src_v (all heads, all slots).  The pairs come from pa_seq_swap_out
 * (device pool -> host pool) or pa_seq_swap_in (host pool -> device pool).
 * src_k/src_v:  [src_num_blocks][H_kv][bs][D], dst_k/dst_v:
 *   [dst_num_blocks][H_kv][bs][D]; block_size, num_kv_heads, head_dim and
 *   dtype come from desc (its num_blocks is not used).  Either pair may be
 *   pinned host memory the GPU can address (hipHostMalloc, torch
 *   pin_memory=True); the other is device memory.
 * src_dst_pairs: int32 [num_pairs][2], device memory or pinned host memory.
 *   Destinations must be distinct; ids outside a pool are skipped.
 * Asynchronous on stream; num_pairs == 0 enqueues nothing.  The caller
 * orders it before any reuse of the source blocks (stream order). */
pa_status pa_swap_blocks(const int32_t* src_dst_pairs, int32_t num_pairs, const void* src_k,
                         const void* src_v, int32_t src_num_blocks, void* dst_k, void* dst_v,
                         int32_t dst_num_blocks, const pa_cache_desc* desc, void* stream);

/* Single-query (decode) attention through the block tables [P1 body: the
 * kernel derives each token's logical block and offset, looks up the
 * physical block and reads K/V there without first gathering the sequence;
 * P3 Step 3; P2 Example: the attention arithmetic is unchanged].
 *
 * For every sequence b < num_seqs and query head h < num_q_heads, with
 * G = num_q_heads / num_kv_heads, kvh = h / G, L = context_lens[b]:
 *   s_p      = scale * dot(q[b][h], K(b, p, kvh))          for p < L
 *   out[b][h] = sum_p softmax(s)_p * V(b, p, kvh)
 * where K(b, p, kvh) = k_cache[block_tables[b][p / bs]][kvh][p % bs][:].
 * L == 0 gives a zero row.  Arithmetic in fp32, one rounding to the output
 * dtype (= pool dtype).
 * q:            device [num_seqs][num_q_heads][head_dim], pool dtype.
 * block_tables: device int32 [num_seqs][max_blocks_per_seq].
 * context_lens: device int32 [num_seqs].
 * block_size:   must equal desc->block_size.
 * out:          device [num_seqs][num_q_heads][head_dim], pool dtype.
 * workspace:    device scratch of at least pa_decode_workspace_size() bytes,
 *               256-byte aligned, ZERO-FILLED before its first use (for
 *               instance by hipMemset or torch.zeros); every call leaves it
 *               ready for the next one (its arrival counters back at zero),
 *               so one zero fill serves any number of calls, graph replays
 *               included, and a workspace sized for num_seqs = B serves
 *               every call of the same head shape with num_seqs <= B.
 *               The call owns it until the stream reaches the end
 *               of the call; calls that share a workspace must be ordered
 *               (one stream, or events): overlapping calls race.
 * num_seqs:     at most 8192 (PA_ERR_UNSUPPORTED beyond, or when the lengths
 *               snapshot would not fit in LDS); num_kv_heads at most 4096.
 * One kernel launch.  The (KV head, sequence, 16-token tile) units are split
 * over the grid in equal shares, dealt so that each XCD takes consecutive
 * shares.  A sequence cut by a share boundary leaves partial results (max,
 * sum, unnormalised output) in the workspace; the last workgroup to finish
 * a piece of it merges them (out = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M)
 * l_i, M = max_i m_i), so no workgroup waits for another. */
pa_status pa_decode(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t num_seqs, int32_t block_size,
                    float scale, void* out, int32_t num_q_heads, const pa_cache_desc* desc,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Appends each sequence's newest token and attends over the result, in one
 * kernel launch: "What is paged attention in vLLM, and why does it
 * matter?", Step 4 (a generated token's K and V go to the next slot of the
 * sequence's last block) followed by Step 3 (attention reads every position
 * through the block table).  The result equals pa_cache_append of the B
 * rows at the slots of positions L_b - 1 (slot = table[b][(L_b - 1) / bs]
 * * bs + (L_b - 1) % bs), then pa_decode with the same arguments: the pools
 * hold the same bytes and the output is bit-identical.
 * new_k, new_v: device [num_seqs][num_kv_heads][head_dim], pool dtype,
 *               16-byte aligned: K and V of the token at position L_b - 1
 *               of sequence b (context_lens counts it).  A sequence with
 *               L_b = 0 appends nothing; a block id outside the pool is
 *               read clamped (output unspecified, as for pa_decode) and
 *               nothing is written there.
 * k_cache, v_cache: written at those slots only (the caller has done any
 *               copy-on-write first, so each written block is private).
 * Every other argument, the workspace and the errors as for pa_decode. */
pa_status pa_decode_append(const void* q, const void* new_k, const void* new_v, void* k_cache,
                           void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t num_seqs, int32_t block_size,
                           float scale, void* out, int32_t num_q_heads, const pa_cache_desc* desc,
                           void* workspace, size_t workspace_bytes, void* stream);

/* pa_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments and result as pa_decode without the workspace, which
 * is a 21 MiB array the library keeps on each GPU until the process ends
 * (its address is looked up once per device; no hipMalloc, hipFree or
 * other allocating call is made).  Its first 4 MiB hold the arrival
 * counters (8 bytes per (sequence, KV head): num_seqs * num_kv_heads at
 * most 524288), the other 17 MiB the partial results (2048 slots of
 * G * (head_dim + 2) floats, G = num_q_heads / num_kv_heads: G * (head_dim
 * + 2) at most 2176, e.g. G = 16 with head_dim 128).  The array starts
 * zero-filled and every call leaves its counters back at zero.  All calls
 * on one GPU share it, so calls that overlap on one GPU (different streams
 * without ordering) race.  PA_ERR_UNSUPPORTED, with nothing launched, when
 * the shape needs more than either region holds. */
pa_status pa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t num_seqs, int32_t block_size,
                            float scale, void* out, int32_t num_q_heads, const pa_cache_desc* desc,
                            void* stream);

/* Causal multi-query attention through the block tables: prefill and
 * chunked prefill [P1 body: prefill allocates and fills a prompt's blocks;
 * P3 Step 3: the prompt's tokens fill logical blocks mapped to scattered
 * physical ones; P2 Example: the attention arithmetic is the ordinary one].
 *
 * Sequence b holds L = context_lens[b] tokens in the cache, the n_b =
 * query_start[b+1] - query_start[b] query tokens included (appended first by
 * pa_cache_append).  Query token i (0 <= i < n_b) is at position
 * p = L - n_b + i and, for every query head h (KV head h / G):
 *   out[query_start[b] + i][h] = sum_{t <= p} softmax(s)_t * V(b, t, kvh),
 *   s_t = scale * dot(q[query_start[b] + i][h], K(b, t, kvh)).
 * q, out:       device [num_query_tokens][num_q_heads][head_dim], the pool
 *               dtype, which must be 16-bit (PA_BF16 or PA_F16;
 *               PA_ERR_UNSUPPORTED for PA_F32).
 * query_start:  device int32 [num_seqs + 1], non-decreasing from 0 to
 *               num_query_tokens (values are clamped into that range; n_b is
 *               clamped to [0, L]; L to max_blocks_per_seq * block_size).
 * block_tables, context_lens, block_size, desc: as for pa_decode.
 * num_seqs at most 8192.  No workspace: one workgroup computes each
 * (sequence, KV head, query block of 16-32 tokens) over its whole causal key
 * range, longest sequences first when num_seqs <= 256.  n_b == 1 for every
 * sequence is decode.  num_query_tokens == 0 enqueues nothing. */
pa_status pa_prefill(const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, const int32_t* query_start, int32_t num_seqs,
                     int32_t num_query_tokens, int32_t block_size, float scale, void* out,
                     int32_t num_q_heads, const pa_cache_desc* desc, void* stream);

/* pa_prefill with long query blocks split along the keys (same arguments,
 * same result up to fp32 summation order), for calls with few query tokens
 * against long contexts (chunked prefill).  When the call has few query
 * blocks (at most 640 (query block of 16 rows, KV head) items, bounded from
 * num_query_tokens and num_seqs), the key range of each query block is cut
 * into pieces of at least 48 key tiles of 32 keys; each piece is computed by
 * its own workgroup into the workspace (per row: the softmax reference
 * maximum, the sum and the unnormalised output), and a second kernel on the
 * same stream merges the pieces (out = sum_i 2^(m_i - M) o_i /
 * sum_i 2^(m_i - M) l_i, M = max_i m_i).  Otherwise it runs exactly as
 * pa_prefill and leaves the workspace alone.
 * workspace:    device scratch of at least pa_prefill_split_workspace_size()
 *               bytes (0 when the shape is not split; then it may be NULL),
 *               256-byte aligned, needing no initialisation; calls that
 *               share it must be ordered on one stream.
 * The number of pieces is bounded from host-known sizes only (num_seqs,
 * num_query_tokens, max_blocks_per_seq), so the workspace size and the grid
 * depend on them, not on the lengths' values.  query_start must be
 * non-decreasing: with overlapping query ranges pieces past that bound are
 * not computed and their rows are left unwritten (never out of bounds). */
pa_status pa_prefill_split(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, const int32_t* query_start,
                           int32_t num_seqs, int32_t num_query_tokens, int32_t block_size,
                           float scale, void* out, int32_t num_q_heads,
                           const pa_cache_desc* desc, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Bytes of workspace pa_prefill_split needs for this shape (0 when it would
 * not split). */
pa_status pa_prefill_split_workspace_size(const pa_cache_desc* desc, int32_t num_seqs,
                                          int32_t num_q_heads, int32_t num_query_tokens,
                                          int32_t max_blocks_per_seq, size_t* bytes);

/* Bytes of workspace pa_decode needs for this shape (independent of the
 * lengths' values). */
pa_status pa_decode_workspace_size(const pa_cache_desc* desc, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t max_blocks_per_seq,
                                   size_t* bytes);

/* ------------------------------------------------------------ allocator */

/* Host block allocator: a free list, one reference count per block and one
 * block table per sequence [P3 Step 3: the block manager keeps the tables
 * beside a pool of free blocks and per-block reference counts].
 *
 * - Lazy allocation: a sequence takes a block only when a token arrives and
 *   its last block is full [P3 Step 4; P2 How it works, item 2].
 * - Free list: LIFO.  A fresh allocator hands blocks out in free_order
 *   (a permutation of 0..num_blocks-1; NULL = ascending).  pa_seq_free
 *   pushes a sequence's blocks in reverse logical order, so its logical
 *   block 0 is handed out first afterwards [P3 Step 4: freed blocks can be
 *   taken by other requests at once].
 * - Fork shares every block of the parent (count + 1) [P2 How it works,
 *   item 4].
 * - Copy-on-write: a token written into a partly filled block with count > 1
 *   first moves the writer to a fresh block and reports (src, dst) for
 *   pa_copy_blocks [P2 How it works, item 5].  Sequences are processed in
 *   call order, so the last remaining sharer writes in place.  A full shared
 *   block is never copied (the next token takes a fresh block).
 * - Every call gives the strong guarantee: on any error nothing changed.
 * - Preemption [P1 Common questions and P3 Follow-up questions, on running
 *   out of blocks]: an optional pool of host blocks with its own LIFO stack.
 *   Swap-out moves a whole sequence to host blocks and releases its device
 *   blocks as a free does (shared blocks stay with the other sharers);
 *   swap-in moves it back into private device blocks.  Drop-and-recompute
 *   needs no new call: pa_seq_free, pa_seq_create, pa_seq_reserve, then
 *   append and prefill.
 * Handles are owned by the caller (create/destroy); not thread-safe. */
typedef struct pa_allocator pa_allocator;

pa_status pa_allocator_create(int32_t num_blocks, int32_t block_size,
                              const int32_t* free_order /* host, nullable */,
                              pa_allocator** out);
void pa_allocator_destroy(pa_allocator* alloc);

/* New empty sequence.  INVALID_ARGUMENT if the id exists. */
pa_status pa_seq_create(pa_allocator* alloc, int64_t seq_id);

/* child := copy of parent's table and length; each block's count + 1.
 * UNKNOWN_SEQ if parent is absent, INVALID_ARGUMENT if child exists. */
pa_status pa_seq_fork(pa_allocator* alloc, int64_t parent, int64_t child);

/* Gives n_new[i] new tokens to seq_ids[i] for i < n, in that order.
 * slot_mapping_out: host int64 [sum(n_new)], sequence-major in call order.
 * cow_pairs_out:    host int32 [cow_cap][2] (src, dst); *num_cow_out = count.
 * Errors (checked in order for each i before any change): n_new[i] < 0 or a
 * repeated id -> INVALID_ARGUMENT; unknown id -> UNKNOWN_SEQ.  Running out of
 * blocks -> OUT_OF_BLOCKS, more pairs than cow_cap -> INVALID_ARGUMENT; both
 * leave the allocator exactly as before the call (all-or-nothing). */
pa_status pa_seq_reserve(pa_allocator* alloc, const int64_t* seq_ids, const int32_t* n_new,
                         int32_t n, int64_t* slot_mapping_out, int32_t* cow_pairs_out,
                         int32_t cow_cap, int32_t* num_cow_out);

/* Drops the sequence; blocks whose count reaches zero rejoin the free list. */
pa_status pa_seq_free(pa_allocator* alloc, int64_t seq_id);

/* tables_out: host int32 [n][max_blocks_per_seq] padded with -1;
 * context_lens_out: host int32 [n].  INVALID_ARGUMENT if a table is longer
 * than max_blocks_per_seq, UNKNOWN_SEQ for an absent id. */
pa_status pa_build_block_tables(const pa_allocator* alloc, const int64_t* seq_ids, int32_t n,
                                int32_t max_blocks_per_seq, int32_t* tables_out,
                                int32_t* context_lens_out);

/* Snapshot getters (host memory). */
int32_t pa_allocator_num_free(const pa_allocator* alloc);
/* Free blocks, the one handed out next first; *len = count, at most cap
 * written (INVALID_ARGUMENT if cap is too small, nothing written). */
pa_status pa_allocator_free_list(const pa_allocator* alloc, int32_t* out, int32_t cap,
                                 int32_t* len);
pa_status pa_block_refcount(const pa_allocator* alloc, int32_t block, int32_t* out);
pa_status pa_seq_block_table(const pa_allocator* alloc, int64_t seq_id, int32_t* out,
                             int32_t cap, int32_t* len);
pa_status pa_seq_num_tokens(const pa_allocator* alloc, int64_t seq_id, int32_t* out);

/* Adds the host block pool: num_host_blocks blocks handed out in free_order
 * (host, a permutation of 0..num_host_blocks-1; NULL = ascending).
 * INVALID_ARGUMENT if the allocator already has one. */
pa_status pa_allocator_add_host_pool(pa_allocator* alloc, int32_t num_host_blocks,
                                     const int32_t* free_order);

/* Moves seq_id to host blocks: one host block per logical block, in logical
 * order, popped from the host stack; pairs_out (host int32 [cap][2]) gets
 * (device block, host block) per logical block for pa_swap_blocks; then the
 * device blocks are released as by pa_seq_free (reverse logical order,
 * pushed when their count reaches zero).  The sequence's table then holds
 * host block ids; its length is unchanged.  Errors, in order: UNKNOWN_SEQ;
 * INVALID_ARGUMENT if already swapped out or there is no host pool;
 * OUT_OF_BLOCKS if the host pool is short; INVALID_ARGUMENT if cap is below
 * the table length.  Each leaves the allocator unchanged. */
pa_status pa_seq_swap_out(pa_allocator* alloc, int64_t seq_id, int32_t* pairs_out, int32_t cap,
                          int32_t* num_pairs_out);

/* Moves a swapped-out sequence back: one device block (count 1) per logical
 * block from the device stack; pairs_out gets (host block, device block);
 * then the host blocks return to the host stack in reverse logical order.
 * Errors, in order: UNKNOWN_SEQ; INVALID_ARGUMENT if not swapped out;
 * OUT_OF_BLOCKS if the device pool is short; INVALID_ARGUMENT if cap is too
 * small.  A swapped-out sequence cannot be reserved, forked or put in a
 * block table (INVALID_ARGUMENT); pa_seq_free returns its host blocks. */
pa_status pa_seq_swap_in(pa_allocator* alloc, int64_t seq_id, int32_t* pairs_out, int32_t cap,
                         int32_t* num_pairs_out);

/* Automatic prefix caching [P3 Trade-offs and edge cases, fourth point: full
 * blocks are hashed and the least recently used are evicted; P1 Common
 * questions: cached prefixes may be evicted under memory pressure].
 * Turns it on (idempotent).  From then on a block whose count drops to zero
 * and that holds a key waits on an LRU list instead of the free list; a
 * block request takes the free list first, then evicts the least recently
 * released cached block (its key is dropped). */
pa_status pa_allocator_enable_prefix_cache(pa_allocator* alloc);

/* Registers the token ids of an empty sequence (normally its prompt) and
 * takes the cached blocks of its longest cached prefix.  Full block i of
 * tokens has the key FNV-1a-64(key(i-1) as 8 little-endian bytes, then its
 * bs token ids as 4-byte little-endian integers), key(-1) = 0; a hit also
 * matches the stored parent key and token ids.  At most (n - 1) / bs blocks
 * are taken (at least one token is left to compute), in order from block 0
 * up to the first miss; each taken block's count + 1 (off the LRU list if it
 * was 0).  The sequence's length becomes the tokens they hold
 * (*num_cached_out); the caller reserves and fills the rest, and each
 * registered block is cached when a reserve fills it (the first block to
 * hold a key keeps it).  tokens: host int32 [n].  Errors: UNKNOWN_SEQ;
 * INVALID_ARGUMENT if the cache is off or the sequence is not empty. */
pa_status pa_seq_match_prefix(pa_allocator* alloc, int64_t seq_id, const int32_t* tokens,
                              int32_t n, int32_t* num_cached_out);

/* Evictable cached blocks (count 0), and their list, the one evicted next
 * first (as pa_allocator_free_list). */
int32_t pa_allocator_num_cached(const pa_allocator* alloc);
pa_status pa_allocator_cached_list(const pa_allocator* alloc, int32_t* out, int32_t cap,
                                   int32_t* len);

/* Whether block `block` holds a prefix-cache key (in use or evictable), and
 * that key (0 when it holds none or the cache is off).  For bit-exact
 * comparisons of the cache's state.  INVALID_ARGUMENT for a block outside
 * the pool. */
pa_status pa_block_prefix_key(const pa_allocator* alloc, int32_t block, int32_t* cached_out,
                              uint64_t* key_out);

/* *out = 1 if seq_id is swapped out, else 0. */
pa_status pa_seq_is_swapped(const pa_allocator* alloc, int64_t seq_id, int32_t* out);
/* Free host blocks (-1 without a host pool), and the host stack, the block
 * handed out next first (as pa_allocator_free_list). */
int32_t pa_allocator_num_free_host(const pa_allocator* alloc);
pa_status pa_allocator_host_free_list(const pa_allocator* alloc, int32_t* out, int32_t cap,
                                      int32_t* len);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
