// Multi-query (prefill / chunked prefill) attention that reads K/V through
// per-sequence block tables (gfx950 / CDNA4, wave64).
//
// Sources: "Paged Attention" (klaylearn.com glossary), body: prefill
// allocates and fills a prompt's blocks, and the kernel finds every token's
// K/V through the table; "What is paged attention in vLLM, and why does it
// matter?" (interview.clozo.ai), Step 3: the prompt's tokens fill logical
// blocks, mapped to scattered physical blocks; "PagedAttention - AI
// Glossary" (modelrefs.com), Example: the attention arithmetic is the
// ordinary one.  Sequence b holds L_b tokens in the cache; its n_b query
// tokens are the last n_b, the i-th at position L_b - n_b + i, and attends to
// positions 0..L_b - n_b + i (causal).
//
// Work decomposition: a work item is one (sequence, KV head, query tile):
// 16 query rows, i.e. 16 / GP tokens x the GP heads of the KV head's group
// (GP = G rounded up to a power of two; rows of heads >= G are padding).
// One wave takes one item and walks its whole causal key range, 16 keys per
// tile, in batches of NBUF tiles whose loads are all issued before the first
// use.  Items of a sequence are ordered longest first, so the long ones
// start early and the hardware scheduler back-fills the rest.
//
// Per tile: S = K Q^T by v_mfma_f32_16x16x32_bf16 (A = 16 K rows, B = the
// 16 query rows), the lazily rescaled online softmax, and O += P V, l += P 1
// by v_mfma_f32_16x16x16_bf16; the step is the decode kernel's, with a
// causal limit per query row.  Only tiles that cross the diagonal of the
// item's first query token mask anything.
//
// The query rows need MFMA operands in bf16, so the call takes bf16 pools
// only.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>

#include "pa_attn_tile.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace {

using pa::bf16x2_t;
using pa::f32x2_t;
using pa::floatx4_t;
using pa::Geometry;
using pa::kTile;
using pa::kWave;
using pa::MfmaState;
using pa::TileRegs;
using pa::u32x4_t;
using pa::uni;

constexpr int kNW = 4;              // waves per workgroup (one work item each)
constexpr int kMaxSeqs = 8192;      // query starts and lengths snapshot in LDS
constexpr int kChunk = 64;          // table lanes per block-id chunk
#ifndef PA_PREFILL_NB
#define PA_PREFILL_NB 4             // tiles per batch (divides every chunk)
#endif

struct PrefillArgs {
  const void* q;            // [T][H_q][D]
  const int32_t* tables;    // [B][max_blocks]
  const int32_t* lens;      // [B]
  const int32_t* qstart;    // [B + 1]
  void* out;                // [T][H_q][D]
  pa::KvPool pool;
  int32_t B;
  int32_t T;
  int32_t max_blocks;
  int32_t G;
  float scale_log2;         // scale * log2(e)
};

// Largest b in [0, B) with P[b] * H <= f (P: exclusive prefix sums in LDS).
__device__ __forceinline__ int32_t find_item_seq(const int32_t* P, int32_t B, int32_t H,
                                                 int32_t f) {
  int32_t lo = 0, hi = B - 1;
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if (P[mid] * H <= f) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

template <int D, int GP, bool kSmall>
__global__ void __launch_bounds__(kNW * kWave)
prefill_kernel(PrefillArgs a) {
  using Geo = Geometry<true, D>;
  constexpr int kBlk = D / 16;
  constexpr int TP = kTile / GP;  // query tokens per work item
  constexpr int NBUF = PA_PREFILL_NB;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), v = tid >> 6;
  const int jr = lane >> 4, c16 = lane & 15;
  const int32_t B = a.B, H_kv = a.pool.H_kv, G = a.G, H_q = H_kv * G;
  const int log2_bs = a.pool.log2_bs;

  // LDS: per sequence the query start, the number of query tokens n_b
  // (clamped to [0, L_b]) and the exclusive prefix sums of its tiles.
  int32_t* QS = reinterpret_cast<int32_t*>(smem);  // [B]
  int32_t* NQ = QS + B;                            // [B]
  int32_t* PQ = NQ + B;                            // [B + 1]
  int32_t* misc = PQ + B + 1;                      // [kNW]
  const int32_t len_cap = a.max_blocks << log2_bs;
  int32_t carry = 0;
  for (int32_t c = 0; c < B; c += kNW * kWave) {
    const int32_t b = c + tid;
    int32_t nt = 0;
    if (b < B) {
      const int32_t q0 = min(max(a.qstart[b], 0), a.T);
      const int32_t q1 = min(max(a.qstart[b + 1], q0), a.T);
      const int32_t L = min(max(a.lens[b], 0), len_cap);
      const int32_t n = min(q1 - q0, L);
      QS[b] = q0;
      NQ[b] = n;
      nt = (n + TP - 1) / TP;
    }
    const int32_t incl = pa::wave_incl_scan(nt);
    if (lane == kWave - 1) misc[v] = incl;
    __syncthreads();
    int32_t pre = carry, tot = 0;
#pragma unroll
    for (int u = 0; u < kNW; ++u) {
      const int32_t x = misc[u];
      pre += u < v ? x : 0;
      tot += x;
    }
    if (b < B) PQ[b] = pre + incl - nt;
    carry += tot;
    __syncthreads();
  }
  if (tid == 0) PQ[B] = carry;
  __syncthreads();

  // ---- this wave's work item: (b, kvh, query tile qt), longest first
  const int32_t items = uni(PQ[B]) * H_kv;
  const int32_t f = blockIdx.x * kNW + v;
  if (f >= items) return;
  const int32_t b = uni(find_item_seq(PQ, B, H_kv, f));
  const int32_t local = f - uni(PQ[b]) * H_kv;
  const int32_t kvh = local % H_kv;
  const int32_t nq = uni(NQ[b]);
  const int32_t nqt = (nq + TP - 1) / TP;
  const int32_t qt = nqt - 1 - local / H_kv;
  const int32_t L = min(max(a.lens[b], 0), len_cap);  // wave-uniform (scalar load)
  const int32_t i0 = qt * TP, i1 = min(i0 + TP, nq);  // query tokens [i0, i1)
  const int32_t pbase = L - nq;                        // position of query token 0
  const int32_t p_min = pbase + i0, p_max = pbase + i1 - 1;
  const int32_t nkv = (p_max + kTile) / kTile;          // key tiles 0 .. p_max

  // Query rows: lane c16 is row c16 = (token i0 + c16 / GP, head c16 % GP);
  // padding rows (past the item's tokens, or heads >= G) are zero.
  const int32_t row_i = i0 + c16 / GP, row_g = c16 % GP;
  const bool row_live = row_i < i1 && row_g < G;
  const int32_t lim = row_live ? pbase + row_i : p_max;  // causal limit of this lane's row
  u32x4_t qf[Geo::kQRegs];
  {
    const int32_t qs_b = uni(QS[b]);
    const int64_t row = ((int64_t)(qs_b + (row_live ? row_i : i0)) * H_q + kvh * G +
                         (row_live ? row_g : 0));
    const char* qb = reinterpret_cast<const char*>(a.q) + row * Geo::kRowBytes + jr * 16;
#pragma unroll
    for (int p = 0; p < Geo::kKPieces; ++p) {
      u32x4_t x = *reinterpret_cast<const u32x4_t*>(qb + p * 64);
      qf[p] = row_live ? x : u32x4_t{0, 0, 0, 0};
    }
  }

  // ---- block ids, one chunk of kChunk table lanes ahead: lane i of the
  // chunk holding tile kt describes tile tpc * c + i / nbt, sub-block
  // i % nbt (nbt = table lanes per tile).  Entries are clamped into the row.
  const int nbt = log2_bs >= 4 ? 1 : (kTile >> log2_bs);
  const int tpc_log = log2_bs >= 4 ? 6 : 2 + log2_bs;  // log2(tiles per chunk)
  const int32_t* trow = a.tables + (int64_t)b * a.max_blocks;
  auto describe = [&](int32_t c) -> int32_t {
    const int32_t kt = min((c << tpc_log) + lane / nbt, nkv - 1);
    const int32_t tok = min(kt * kTile + ((lane & (nbt - 1)) << log2_bs), L - 1);
    return trow[min(tok >> log2_bs, a.max_blocks - 1)];
  };
  int32_t cur = describe(0), nxt = describe(1);
  int32_t cur_c = 0;

  MfmaState<D> st;
  st.reset();
  for (int32_t k0 = 0; k0 < nkv; k0 += NBUF) {
    // A batch never straddles a chunk (NBUF divides the tiles per chunk).
    const int32_t c = k0 >> tpc_log;
    if (c != cur_c) {
      cur = nxt;
      cur_c = c;
      nxt = describe(c + 1);
    }
    TileRegs<true, D> buf[NBUF];
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {
      const int32_t kt = min(k0 + u, nkv - 1);
      const int32_t jl = kt - (c << tpc_log);
      if constexpr (kSmall) {
        pa::issue_tile_small<true, D>(buf[u], a.pool, cur, jl, kt, kvh, L, nbt, lane);
      } else {
        const int32_t phys = __builtin_amdgcn_readlane(cur, jl);
        pa::issue_tile<true, D>(buf[u], a.pool, phys, kt, kvh, lane, k0 + u < nkv);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    pa::static_for<0, NBUF>([&](auto U) {
      constexpr int u = decltype(U)::value;
      const int32_t t0 = (k0 + u) * kTile;
      if (k0 + u < nkv) {
        if (t0 + kTile - 1 <= p_min)  // every key at or before every live row
          pa::consume_tile_mfma_impl<D, false>(st, buf[u], qf, a.scale_log2, t0, lim, L, lane);
        else
          pa::consume_tile_mfma_impl<D, true>(st, buf[u], qf, a.scale_log2, t0, lim, L, lane);
      }
    });
  }

  // ---- finish: lane 16j + c, register r holds row 4j + r, columns
  // kBlk * c .. kBlk * c + kBlk - 1; its normaliser is st.l[r].
  pa::static_for<0, 4>([&](auto R) {
    constexpr int r = decltype(R)::value;
    const int row = 4 * jr + r;
    const int32_t i = i0 + row / GP, g = row % GP;
    if (i < i1 && g < G) {
      const float inv = 1.f / st.l[r];
      uint32_t pk[kBlk / 2];
#pragma unroll
      for (int k = 0; k < kBlk / 2; ++k) {
        const f32x2_t pr = {st.acc[2 * k][r] * inv, st.acc[2 * k + 1][r] * inv};
        pk[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2_t));
      }
      char* dst = reinterpret_cast<char*>(a.out) +
                  (((int64_t)(uni(QS[b]) + i) * H_q + kvh * G + g) * D + kBlk * c16) * 2;
      if constexpr (kBlk == 8) *reinterpret_cast<u32x4_t*>(dst) = u32x4_t{pk[0], pk[1], pk[2], pk[3]};
      else *reinterpret_cast<uint2*>(dst) = uint2{pk[0], pk[1]};
    }
  });
}

template <int D, int GP>
pa_status launch(const PrefillArgs& a, hipStream_t s) {
  constexpr int TP = kTile / GP;
  auto kern = a.pool.log2_bs >= 4 ? prefill_kernel<D, GP, false> : prefill_kernel<D, GP, true>;
  // Work items: at most ceil(T / TP) + B query tiles per KV head; the kernel
  // numbers them in int32.
  const int64_t items = (((int64_t)a.T + TP - 1) / TP + a.B) * a.pool.H_kv;
  if (items + kNW >= (1ll << 31))
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_prefill: too many query tiles");
  const int64_t wgs = (items + kNW - 1) / kNW;
  const size_t lds = (size_t)(3 * a.B + 1 + kNW) * sizeof(int32_t);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess)
      return pa::fail(PA_ERR_DEVICE, "pa_prefill: LDS attribute: %s", hipGetErrorString(e));
  }
  hipLaunchKernelGGL(kern, dim3((uint32_t)wgs), dim3(kNW * kWave), lds, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pa::fail(PA_ERR_DEVICE, "pa_prefill: %s", hipGetErrorString(e));
  return PA_OK;
}

template <int D>
pa_status dispatch_g(const PrefillArgs& a, hipStream_t s) {
  if (a.G <= 1) return launch<D, 1>(a, s);
  if (a.G <= 2) return launch<D, 2>(a, s);
  if (a.G <= 4) return launch<D, 4>(a, s);
  if (a.G <= 8) return launch<D, 8>(a, s);
  return launch<D, 16>(a, s);
}

}  // namespace

extern "C" {

pa_status pa_prefill(const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, const int32_t* query_start, int32_t num_seqs,
                     int32_t num_query_tokens, int32_t block_size, float scale, void* out,
                     int32_t num_q_heads, const pa_cache_desc* desc, void* stream) {
  pa_status st = pa_supported(desc, num_q_heads);
  if (st != PA_OK) return st;
  if (desc->dtype != PA_BF16)
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_prefill: bf16 pools only");
  if (block_size != desc->block_size)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "block_size %d != desc->block_size %d", block_size,
                    desc->block_size);
  if (num_seqs < 0 || num_query_tokens < 0 || max_blocks_per_seq < 1)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "num_seqs %d / num_query_tokens %d / "
                    "max_blocks_per_seq %d", num_seqs, num_query_tokens, max_blocks_per_seq);
  if (num_seqs > kMaxSeqs)
    return pa::fail(PA_ERR_UNSUPPORTED, "num_seqs %d > %d", num_seqs, kMaxSeqs);
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "max_blocks_per_seq * block_size overflows int32");
  if (!std::isfinite(scale)) return pa::fail(PA_ERR_INVALID_ARGUMENT, "scale is not finite");
  if (num_seqs == 0 || num_query_tokens == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start || !out)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (!pa::aligned(q, 16) || !pa::aligned(k_cache, 16) || !pa::aligned(v_cache, 16) ||
      !pa::aligned(out, 16) || !pa::aligned(block_tables, 4) || !pa::aligned(context_lens, 4) ||
      !pa::aligned(query_start, 4))
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "misaligned pointer");
  PrefillArgs a;
  a.q = q;
  a.tables = block_tables;
  a.lens = context_lens;
  a.qstart = query_start;
  a.out = out;
  a.pool = pa::KvPool{k_cache, v_cache, desc->num_blocks, desc->num_kv_heads,
                      pa::ilog2_exact(block_size)};
  a.B = num_seqs;
  a.T = num_query_tokens;
  a.max_blocks = max_blocks_per_seq;
  a.G = num_q_heads / desc->num_kv_heads;
  a.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  hipStream_t s = (hipStream_t)stream;
  if (desc->head_dim == 128) return dispatch_g<128>(a, s);
  return dispatch_g<64>(a, s);
}

}  // extern "C"
