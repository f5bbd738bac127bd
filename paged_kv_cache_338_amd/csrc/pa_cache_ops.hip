// Slot-mapped append and copy-on-write block copy (gfx950).
//
// Sources: "What is paged attention in vLLM, and why does it matter?"
// (interview.clozo.ai), Step 4: at every decode step the new token's keys
// and values are written into the sequence's last block; "Paged Attention"
// (klaylearn.com glossary), body: prefill fills freshly allocated blocks the
// same way; "PagedAttention - AI Glossary" (modelrefs.com), How it works,
// item 5, and the clozo.ai Trade-offs section: a block shared by several
// sequences is copied only when one of them writes into it, and only that
// block is copied.
//
// Swap ("Paged Attention" glossary, Common questions, and the clozo.ai page,
// Follow-up questions, on running out of blocks): a preempted sequence's
// blocks move to CPU memory and back.  pa_swap_blocks moves whole blocks
// between two pools of one geometry, either of which may be pinned host
// memory the GPU reads and writes directly (one launch for any scattered
// set of blocks; over the host link the transfer is bound by the link).
//
// All kernels are pure data movement: 16-byte loads and stores, one
// workgroup per token (append) or per (pair, pool, 4 KiB chunk) (block
// moves).
// Out-of-pool slots and block ids are skipped, so a bad index never turns
// into a wild write.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pa_device.h"
#include "pa_internal.h"

namespace {

__global__ void __launch_bounds__(256)
cache_append_kernel(const uint4* __restrict__ k, const uint4* __restrict__ v,
                    const int64_t* __restrict__ slots, uint4* __restrict__ k_cache,
                    uint4* __restrict__ v_cache, int64_t num_slots, int32_t bs, int32_t heads,
                    int32_t row_vecs) {
  const int64_t t = blockIdx.x;
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot / bs;
  const int32_t off = static_cast<int32_t>(slot - blk * bs);
  const int32_t per = heads * row_vecs;
  for (int32_t i = threadIdx.x; i < 2 * per; i += blockDim.x) {
    const bool is_v = i >= per;
    const int32_t j = is_v ? i - per : i;
    const int32_t h = j / row_vecs, c = j - h * row_vecs;
    const uint4 x = (is_v ? v : k)[t * per + j];
    (is_v ? v_cache : k_cache)[((blk * heads + h) * bs + off) * row_vecs + c] = x;
  }
}

// Block src of the source pools -> block dst of the destination pools
// (the same pools for a copy-on-write copy); blockIdx.y picks K or V and
// blockIdx.z a 4 KiB chunk of the block: each thread moves one 16-byte
// vector per chunk, striding by gridDim.z chunks when a block has more than
// the grid's 65,535.  One vector per thread, many small workgroups: on the
// prefix-sharing batch's 127 copy-on-write pairs this moves the 16.6 MB in
// about 3.3 us, where 2-8 vectors per thread (in one or two dependent
// rounds) took 5.7-17 us.
__global__ void __launch_bounds__(256)
move_blocks_kernel(const int32_t* __restrict__ pairs, const uint4* src_k, const uint4* src_v,
                   int32_t src_blocks, uint4* dst_k, uint4* dst_v, int32_t dst_blocks,
                   int64_t block_vecs) {
  const int32_t src = pairs[2 * blockIdx.x], dst = pairs[2 * blockIdx.x + 1];
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  const uint4* s = (blockIdx.y ? src_v : src_k) + src * block_vecs;
  uint4* d = (blockIdx.y ? dst_v : dst_k) + dst * block_vecs;
  for (int64_t i = (int64_t)blockIdx.z * 256 + threadIdx.x; i < block_vecs;
       i += (int64_t)gridDim.z * 256)
    d[i] = s[i];
}

// Grid of move_blocks_kernel for num_pairs pairs of blocks of block_vecs
// 16-byte vectors.
dim3 move_grid(int32_t num_pairs, int64_t block_vecs) {
  const int64_t chunks = (block_vecs + 255) / 256;
  return dim3((uint32_t)num_pairs, 2, (uint32_t)(chunks < 65535 ? chunks : 65535));
}

pa_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pa::fail(PA_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_cache_append(const void* k, const void* v, const int64_t* slot_mapping,
                          int32_t num_tokens, void* k_cache, void* v_cache,
                          const pa_cache_desc* desc, void* stream) {
  pa_status st = pa::check_desc(desc);
  if (st != PA_OK) return st;
  if (num_tokens < 0) return pa::fail(PA_ERR_INVALID_ARGUMENT, "num_tokens %d < 0", num_tokens);
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (!pa::aligned(k, 16) || !pa::aligned(v, 16) || !pa::aligned(k_cache, 16) ||
      !pa::aligned(v_cache, 16) || !pa::aligned(slot_mapping, 8))
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "misaligned pointer");
  const int32_t row_vecs = desc->head_dim * pa::elem_bytes(desc->dtype) / 16;
  hipLaunchKernelGGL(cache_append_kernel, dim3(num_tokens), dim3(256), 0, (hipStream_t)stream,
                     (const uint4*)k, (const uint4*)v, slot_mapping, (uint4*)k_cache,
                     (uint4*)v_cache, (int64_t)desc->num_blocks * desc->block_size,
                     desc->block_size, desc->num_kv_heads, row_vecs);
  return check_launch("pa_cache_append");
}

pa_status pa_copy_blocks(const int32_t* src_dst_pairs, int32_t num_pairs, void* k_cache,
                         void* v_cache, const pa_cache_desc* desc, void* stream) {
  pa_status st = pa::check_desc(desc);
  if (st != PA_OK) return st;
  if (num_pairs < 0) return pa::fail(PA_ERR_INVALID_ARGUMENT, "num_pairs %d < 0", num_pairs);
  if (num_pairs == 0) return PA_OK;
  if (!src_dst_pairs || !k_cache || !v_cache)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (!pa::aligned(k_cache, 16) || !pa::aligned(v_cache, 16) || !pa::aligned(src_dst_pairs, 4))
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "misaligned pointer");
  if (num_pairs > desc->num_blocks)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "num_pairs %d > num_blocks %d", num_pairs,
                    desc->num_blocks);
  const int64_t block_vecs = (int64_t)desc->num_kv_heads * desc->block_size * desc->head_dim *
                             pa::elem_bytes(desc->dtype) / 16;
  hipLaunchKernelGGL(move_blocks_kernel, move_grid(num_pairs, block_vecs), dim3(256), 0,
                     (hipStream_t)stream, src_dst_pairs, (const uint4*)k_cache, (const uint4*)v_cache,
                     desc->num_blocks, (uint4*)k_cache, (uint4*)v_cache, desc->num_blocks,
                     block_vecs);
  return check_launch("pa_copy_blocks");
}

pa_status pa_swap_blocks(const int32_t* src_dst_pairs, int32_t num_pairs, const void* src_k,
                         const void* src_v, int32_t src_num_blocks, void* dst_k, void* dst_v,
                         int32_t dst_num_blocks, const pa_cache_desc* desc, void* stream) {
  pa_status st = pa::check_desc(desc);
  if (st != PA_OK) return st;
  if (num_pairs < 0) return pa::fail(PA_ERR_INVALID_ARGUMENT, "num_pairs %d < 0", num_pairs);
  if (src_num_blocks < 1 || dst_num_blocks < 1)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "src_num_blocks %d / dst_num_blocks %d",
                    src_num_blocks, dst_num_blocks);
  if (num_pairs == 0) return PA_OK;
  if (!src_dst_pairs || !src_k || !src_v || !dst_k || !dst_v)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (!pa::aligned(src_k, 16) || !pa::aligned(src_v, 16) || !pa::aligned(dst_k, 16) ||
      !pa::aligned(dst_v, 16) || !pa::aligned(src_dst_pairs, 4))
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "misaligned pointer");
  if (num_pairs > dst_num_blocks)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "num_pairs %d > dst_num_blocks %d", num_pairs,
                    dst_num_blocks);
  const int64_t block_vecs = (int64_t)desc->num_kv_heads * desc->block_size * desc->head_dim *
                             pa::elem_bytes(desc->dtype) / 16;
  hipLaunchKernelGGL(move_blocks_kernel, move_grid(num_pairs, block_vecs), dim3(256), 0,
                     (hipStream_t)stream, src_dst_pairs, (const uint4*)src_k, (const uint4*)src_v, src_num_blocks,
                     (uint4*)dst_k, (uint4*)dst_v, dst_num_blocks, block_vecs);
  return check_launch("pa_swap_blocks");
}

}  // extern "C"
