// Device half of the paged KV cache library for gfx950 (CDNA4, wave64):
// slot-mapped append, copy-on-write block copy and single-query decode
// attention that reads K/V through per-sequence block tables.
//
// Sources: "Paged Attention" (klaylearn.com glossary), body: the kernel
// turns a token position into (logical block, offset), looks the physical
// block up in the sequence's table and reads K/V there; "What is paged
// attention in vLLM, and why does it matter?" (interview.clozo.ai), Step 3
// (the attention kernel follows the table) and Step 4 (the new token's K/V is
// written into the last block); "PagedAttention - AI Glossary"
// (modelrefs.com), How it works item 5 (copy only the block being written)
// and Example (the attention arithmetic itself is unchanged).
//
// Decode design (one 64-lane wave per work item):
//  * A work item is (sequence, context split, KV head).  Every wave of both
//    decode kernels derives the same split plan from context_lens on the
//    device: split length PART = 16 * ceil(total_tokens / (16 * target)),
//    so the grid size is fixed by the host and independent of the lengths.
//    Split boundaries are logical positions, so the result does not depend
//    on where blocks sit in the pool.
//  * Tokens are processed in tiles of 16.  QK^T for a tile is a dense
//    [16 tokens x D] x [D x G query heads] contraction: one MFMA chain
//    (v_mfma_f32_16x16x32_bf16, or 16x16x4_f32 for fp32 pools) whose
//    operand registers are loaded straight from HBM with 16-byte loads -
//    lane l holds a 16-byte piece of the K row of token (l % 16).
//  * The MFMA result leaves lane 16*j + g with the logits of head g for
//    tokens 4j..4j+3.  Each group of 16 lanes keeps its own online-softmax
//    state (max, sum) for its 4-token slice of every tile, so no cross-lane
//    reduction is needed per tile; the four states are merged once per item.
//  * P*V runs on the VALU in fp32: lane 16*j + c owns D/16 output columns
//    and the V rows of tokens 4j..4j+3 (16-byte loads, 4 rows of 256 B per
//    instruction); the probabilities reach it by DPP row broadcasts.
//  * The next tile's K/V loads are issued before the current tile is
//    consumed (two register buffers).  The table slice of an item is loaded
//    once into a VGPR (lane i = entry i) and read with readlane/bpermute.
//  * Items of sequences with one split write the normalised output; the
//    others write (max, sum, unnormalised o) partials, merged by the second
//    kernel, which also writes the zero rows of empty sequences.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <type_traits>
#include <utility>

#include "pa_internal.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kTile = 16;           // tokens per MFMA tile
constexpr int kTableChunk = 64;     // table entries held in one VGPR

// --------------------------------------------------------------- utilities
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
  // DPP row_newbcast: every lane of a 16-lane row reads lane N of that row.
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       0, __builtin_bit_cast(int, x), 0x150 + N, 0xF, 0xF, false));
}

template <int Begin, int End, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (Begin < End) {
    f(std::integral_constant<int, Begin>{});
    static_for<Begin + 1, End>(f);
  }
}

// Reinterprets one 32-bit word.  Taking the word by value matters: a
// __builtin_bit_cast applied directly to an ext_vector element (v[e]) is
// lowered by this compiler as a cast of element 0 whatever e is.
__device__ __forceinline__ float as_float(uint32_t w) { return __builtin_bit_cast(float, w); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __builtin_bit_cast(float, w & 0xFFFF0000u);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;  // NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ int64_t wave_sum_i64(int64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// ------------------------------------------------------------------- plan
// Split plan shared by both decode kernels.  All lanes return the same
// values.  Lengths are clamped to [0, len_cap].
struct Plan {
  int32_t part;       // tokens per split (multiple of kTile)
  int32_t num_items;  // sum over sequences of ceil(L / part)
};

__device__ __forceinline__ int32_t clamp_len(const int32_t* lens, int b, int32_t len_cap) {
  int32_t L = lens[b];
  return L < 0 ? 0 : (L > len_cap ? len_cap : L);
}

__device__ Plan make_plan(const int32_t* lens, int B, int32_t len_cap, int32_t target, int lane) {
  int64_t tot = 0;
  for (int b = lane; b < B; b += kWave) tot += clamp_len(lens, b, len_cap);
  tot = wave_sum_i64(tot);
  int64_t per = (tot + target - 1) / target;
  int64_t part = ((per + kTile - 1) / kTile) * kTile;
  if (part < kTile) part = kTile;
  if (part > (int64_t)1 << 30) part = (int64_t)1 << 30;
  Plan p;
  p.part = static_cast<int32_t>(part);
  int64_t items = 0;
  for (int b = lane; b < B; b += kWave) items += (clamp_len(lens, b, len_cap) + p.part - 1) / p.part;
  p.num_items = static_cast<int32_t>(wave_sum_i64(items));
  return p;
}

// Finds the sequence b holding global split index w (0 <= w < num_items) and
// the first split index of b.  All lanes return the same values.
__device__ void find_item(const int32_t* lens, int B, int32_t len_cap, int32_t part, int32_t w,
                          int lane, int* b_out, int32_t* first_out) {
  int32_t base = 0;
  for (int c = 0; c < B; c += kWave) {
    int b = c + lane;
    int n = b < B ? (clamp_len(lens, b, len_cap) + part - 1) / part : 0;
    int incl = wave_incl_scan(n, lane);
    int32_t chunk_total = __shfl(incl, kWave - 1);
    if (w < base + chunk_total) {
      uint64_t hit = __ballot(base + incl > w);
      int first = __builtin_ctzll(hit);
      *b_out = c + first;
      *first_out = base + __shfl(incl - n, first);
      return;
    }
    base += chunk_total;
  }
  *b_out = -1;
  *first_out = 0;
}

// --------------------------------------------------------------- append
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

// ------------------------------------------------------------ copy blocks
__global__ void __launch_bounds__(256)
copy_blocks_kernel(const int32_t* __restrict__ pairs, uint4* __restrict__ k_cache,
                   uint4* __restrict__ v_cache, int32_t num_blocks, int64_t block_vecs) {
  const int32_t src = pairs[2 * blockIdx.x], dst = pairs[2 * blockIdx.x + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  uint4* base = blockIdx.y ? v_cache : k_cache;
  const uint4* s = base + src * block_vecs;
  uint4* d = base + dst * block_vecs;
  constexpr int kUnroll = 4;
  int64_t i = threadIdx.x;
  for (; i + (kUnroll - 1) * 256 < block_vecs; i += kUnroll * 256) {
    uint4 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x[u] = s[i + u * 256];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) d[i + u * 256] = x[u];
  }
  for (; i < block_vecs; i += 256) d[i] = s[i];
}

// ----------------------------------------------------------------- decode
struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* tables;
  const int32_t* lens;
  void* out;
  float* ws_o;     // [cap_items][H_kv][G][D]
  float2* ws_ml;   // [cap_items][H_kv][G] (max in log2 units, sum)
  int32_t B;
  int32_t max_blocks;
  int32_t num_blocks;
  int32_t H_kv;
  int32_t G;
  int32_t log2_bs;
  float scale_log2;  // scale * log2(e)
  int32_t target;    // wanted splits per KV head
  int32_t cap_items; // workspace capacity in (sequence, split) items
};

template <bool BF16, int D>
struct Geometry {
  static constexpr int kElem = BF16 ? 2 : 4;
  static constexpr int kRowBytes = D * kElem;
  static constexpr int kKPieces = kRowBytes / 64;     // 16-byte K pieces per lane per tile
  static constexpr int kVWords = kRowBytes / 16 / 4;  // 32-bit words of V per lane per token
  static constexpr int kCols = D / 16;                // output columns per lane
  static_assert(kRowBytes % 64 == 0, "row must be a multiple of 64 bytes");
};

template <bool BF16, int D>
struct TileRegs {
  using Geo = Geometry<BF16, D>;
  u32x4_t k[Geo::kKPieces];
  uint32_t v[4][Geo::kVWords];
};

// Issues the loads of one 16-token tile.  Token t0 + x for x in [0,16) must
// be below `end`, except in the sequence's last tile where rows at or past
// `end` are read from a clamped (valid) position and masked later.
template <bool BF16, int D>
__device__ __forceinline__ void load_tile(TileRegs<BF16, D>& r, const DecodeArgs& a,
                                          const char* kbase, const char* vbase, int32_t t0,
                                          int32_t end, int32_t tab, int32_t chunk_base, int lane,
                                          int kvh) {
  using Geo = Geometry<BF16, D>;
  const int bs_log = a.log2_bs;
  const int32_t bs = 1 << bs_log;
  const int64_t head_stride = (int64_t)bs * Geo::kRowBytes;
  const int64_t block_stride = head_stride * a.H_kv;
  const int jr = lane >> 4, c16 = lane & 15;
  if (bs_log >= 4) {
    // The whole tile lies in one block: one uniform table entry.
    const int32_t lb = t0 >> bs_log;
    int32_t phys = __builtin_amdgcn_readlane(tab, lb - chunk_base);
    phys = min(max(phys, 0), a.num_blocks - 1);
    const int64_t off0 = (int64_t)phys * block_stride + (int64_t)kvh * head_stride +
                         (int64_t)(t0 & (bs - 1)) * Geo::kRowBytes;
    const char* kp = kbase + off0 + (lane & 15) * Geo::kRowBytes + jr * 16;
#pragma unroll
    for (int p = 0; p < Geo::kKPieces; ++p)
      r.k[p] = *reinterpret_cast<const u32x4_t*>(kp + p * 64);
    const char* vp = vbase + off0 + (jr * 4) * Geo::kRowBytes + c16 * (Geo::kVWords * 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (Geo::kVWords == 4) {
        u32x4_t x = *reinterpret_cast<const u32x4_t*>(vp + q * Geo::kRowBytes);
        r.v[q][0] = x[0]; r.v[q][1] = x[1]; r.v[q][2] = x[2]; r.v[q][3] = x[3];
      } else if constexpr (Geo::kVWords == 2) {
        uint2 x = *reinterpret_cast<const uint2*>(vp + q * Geo::kRowBytes);
        r.v[q][0] = x.x; r.v[q][1] = x.y;
      } else {
#pragma unroll
        for (int h = 0; h < Geo::kVWords / 4; ++h) {
          u32x4_t x = *reinterpret_cast<const u32x4_t*>(vp + q * Geo::kRowBytes + h * 16);
          r.v[q][4 * h + 0] = x[0]; r.v[q][4 * h + 1] = x[1];
          r.v[q][4 * h + 2] = x[2]; r.v[q][4 * h + 3] = x[3];
        }
      }
    }
  } else {
    // Blocks smaller than a tile: every lane finds its own token's block.
    auto row_addr = [&](int32_t tok, const char* base) -> const char* {
      tok = min(tok, end - 1);
      const int32_t lb = tok >> bs_log;
      int32_t phys = __shfl(tab, lb - chunk_base);
      phys = min(max(phys, 0), a.num_blocks - 1);
      return base + (int64_t)phys * block_stride + (int64_t)kvh * head_stride +
             (int64_t)(tok & (bs - 1)) * Geo::kRowBytes;
    };
    const char* kp = row_addr(t0 + (lane & 15), kbase) + jr * 16;
#pragma unroll
    for (int p = 0; p < Geo::kKPieces; ++p)
      r.k[p] = *reinterpret_cast<const u32x4_t*>(kp + p * 64);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const char* vp = row_addr(t0 + jr * 4 + q, vbase) + c16 * (Geo::kVWords * 4);
      if constexpr (Geo::kVWords == 4) {
        u32x4_t x = *reinterpret_cast<const u32x4_t*>(vp);
        r.v[q][0] = x[0]; r.v[q][1] = x[1]; r.v[q][2] = x[2]; r.v[q][3] = x[3];
      } else if constexpr (Geo::kVWords == 2) {
        uint2 x = *reinterpret_cast<const uint2*>(vp);
        r.v[q][0] = x.x; r.v[q][1] = x.y;
      } else {
#pragma unroll
        for (int h = 0; h < Geo::kVWords / 4; ++h) {
          u32x4_t x = *reinterpret_cast<const u32x4_t*>(vp + h * 16);
          r.v[q][4 * h + 0] = x[0]; r.v[q][4 * h + 1] = x[1];
          r.v[q][4 * h + 2] = x[2]; r.v[q][4 * h + 3] = x[3];
        }
      }
    }
  }
}

template <bool BF16, int D, int GP>
struct SplitState {
  using Geo = Geometry<BF16, D>;
  float m;                    // lane 16j+g: running max of head g over row j (log2 units)
  float l;                    // lane 16j+g: running sum of exp2(x - m)
  float o[GP][Geo::kCols];    // lane 16j+c: unnormalised output, columns of chunk c
};

// Consumes one tile: logits by MFMA, online softmax per 16-lane row, P*V.
template <bool BF16, int D, int GP>
__device__ __forceinline__ void consume_tile(SplitState<BF16, D, GP>& st,
                                             const TileRegs<BF16, D>& r, const u32x4_t* qf,
                                             const float* qf32, float scale_log2, int32_t t0,
                                             int32_t end, int lane) {
  using Geo = Geometry<BF16, D>;
  floatx4_t s = {0.f, 0.f, 0.f, 0.f};
  if constexpr (BF16) {
#pragma unroll
    for (int p = 0; p < Geo::kKPieces; ++p)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, r.k[p]),
                                                  __builtin_bit_cast(bf16x8_t, qf[p]), s, 0, 0, 0);
  } else {
#pragma unroll
    for (int p = 0; p < Geo::kKPieces; ++p) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        s = __builtin_amdgcn_mfma_f32_16x16x4f32(as_float(r.k[p][e]),
                                                 qf32[4 * p + e], s, 0, 0, 0);
    }
  }
  const int jr = lane >> 4;
  const bool tail = t0 + kTile > end;
  float x[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    x[q] = s[q] * scale_log2;
    if (tail && t0 + jr * 4 + q >= end) x[q] = -INFINITY;
  }
  const float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  const float m_new = fmaxf(st.m, mx);
  const float alpha = exp2f(st.m - m_new);
  float pr[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) pr[q] = exp2f(x[q] - m_new);
  st.l = st.l * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
  st.m = m_new;

  // V rows of this lane's 4 tokens, widened to fp32; rows past `end` are
  // zeroed so that garbage (even NaN) in unused slots cannot leak in.
  float vf[4][Geo::kCols];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bool ok = !tail || (t0 + jr * 4 + q < end);
#pragma unroll
    for (int w = 0; w < Geo::kVWords; ++w) {
      if constexpr (BF16) {
        vf[q][2 * w] = ok ? bf16_lo(r.v[q][w]) : 0.f;
        vf[q][2 * w + 1] = ok ? bf16_hi(r.v[q][w]) : 0.f;
      } else {
        vf[q][w] = ok ? as_float(r.v[q][w]) : 0.f;
      }
    }
  }
  static_for<0, GP>([&](auto gi) {
    constexpr int g = decltype(gi)::value;
    const float a = row_bcast<g>(alpha);
    float p[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) p[q] = row_bcast<g>(pr[q]);
#pragma unroll
    for (int c = 0; c < Geo::kCols; ++c) {
      float acc = st.o[g][c] * a;
#pragma unroll
      for (int q = 0; q < 4; ++q) acc = fmaf(p[q], vf[q][c], acc);
      st.o[g][c] = acc;
    }
  });
}

template <bool BF16, int D, int GP>
__global__ void __launch_bounds__(kWave)
decode_split_kernel(DecodeArgs a) {
  using Geo = Geometry<BF16, D>;
  using T = std::conditional_t<BF16, uint16_t, float>;
  const int lane = threadIdx.x;
  const int32_t len_cap = a.max_blocks << a.log2_bs;
  const Plan plan = make_plan(a.lens, a.B, len_cap, a.target, lane);
  const int32_t total = plan.num_items * a.H_kv;
  const int jr = lane >> 4, c16 = lane & 15;
  const int32_t H_q = a.H_kv * a.G;

  for (int32_t w = blockIdx.x; w < total; w += gridDim.x) {
    const int32_t item = w / a.H_kv;
    const int kvh = w - item * a.H_kv;
    int b;
    int32_t first;
    find_item(a.lens, a.B, len_cap, plan.part, item, lane, &b, &first);
    if (b < 0) break;
    const int32_t L = clamp_len(a.lens, b, len_cap);
    const int32_t split = item - first;
    const int32_t nsplit = (L + plan.part - 1) / plan.part;
    const int32_t start = split * plan.part;
    const int32_t end = min(L, start + plan.part);

    // Query of this KV head's G heads as the MFMA B operand (zero for g >= G).
    u32x4_t qf[BF16 ? Geo::kKPieces : 1];
    float qf32[BF16 ? 1 : Geo::kKPieces * 4];
    {
      const bool live = c16 < a.G;
      const T* qrow = reinterpret_cast<const T*>(a.q) +
                      ((int64_t)b * H_q + (int64_t)kvh * a.G + (live ? c16 : 0)) * D;
      const char* qb = reinterpret_cast<const char*>(qrow) + jr * 16;
#pragma unroll
      for (int p = 0; p < Geo::kKPieces; ++p) {
        u32x4_t x = live ? *reinterpret_cast<const u32x4_t*>(qb + p * 64) : u32x4_t{0, 0, 0, 0};
        if constexpr (BF16) {
          qf[p] = x;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) qf32[4 * p + e] = as_float(x[e]);
        }
      }
    }

    // Hoisted table slice: lane i holds table[b][chunk_base + i].
    const int32_t* trow = a.tables + (int64_t)b * a.max_blocks;
    const int32_t lb_last = (end - 1) >> a.log2_bs;
    int32_t chunk_base = start >> a.log2_bs;
    auto load_chunk = [&](int32_t base) {
      const int32_t i = base + lane;
      return i <= lb_last ? trow[i] : 0;
    };
    int32_t tab = load_chunk(chunk_base);
    auto ensure = [&](int32_t t0) {
      const int32_t hi = min(t0 + kTile, end) - 1;
      if ((hi >> a.log2_bs) >= chunk_base + kTableChunk) {
        chunk_base = t0 >> a.log2_bs;
        tab = load_chunk(chunk_base);
      }
    };

    SplitState<BF16, D, GP> st;
    st.m = -3.0e38f;
    st.l = 0.f;
#pragma unroll
    for (int g = 0; g < GP; ++g)
#pragma unroll
      for (int c = 0; c < Geo::kCols; ++c) st.o[g][c] = 0.f;

    const char* kbase = reinterpret_cast<const char*>(a.k_cache);
    const char* vbase = reinterpret_cast<const char*>(a.v_cache);
    const int32_t ntiles = (end - start + kTile - 1) / kTile;
    TileRegs<BF16, D> ra, rb;
    load_tile(ra, a, kbase, vbase, start, end, tab, chunk_base, lane, kvh);
    for (int32_t i = 0; i < ntiles; i += 2) {
      const int32_t t0 = start + i * kTile;
      if (i + 1 < ntiles) {
        ensure(t0 + kTile);
        load_tile(rb, a, kbase, vbase, t0 + kTile, end, tab, chunk_base, lane, kvh);
      }
      consume_tile(st, ra, qf, qf32, a.scale_log2, t0, end, lane);
      if (i + 2 < ntiles) {
        ensure(t0 + 2 * kTile);
        load_tile(ra, a, kbase, vbase, t0 + 2 * kTile, end, tab, chunk_base, lane, kvh);
      }
      if (i + 1 < ntiles) consume_tile(st, rb, qf, qf32, a.scale_log2, t0 + kTile, end, lane);
    }

    // Merge the four row states: lanes g, 16+g, 32+g, 48+g hold head g.
    float M = fmaxf(st.m, __shfl_xor(st.m, 16));
    M = fmaxf(M, __shfl_xor(M, 32));
    const float sc = exp2f(st.m - M);
    float lt = st.l * sc;
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    static_for<0, GP>([&](auto gi) {
      constexpr int g = decltype(gi)::value;
      const float f = row_bcast<g>(sc);
#pragma unroll
      for (int c = 0; c < Geo::kCols; ++c) {
        float v = st.o[g][c] * f;
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        st.o[g][c] = v;
      }
    });

    if (nsplit == 1) {
      static_for<0, GP>([&](auto gi) {
        constexpr int g = decltype(gi)::value;
        const float inv = 1.f / row_bcast<g>(lt);
        if (g < a.G && (g & 3) == jr) {
          T* orow = reinterpret_cast<T*>(a.out) + ((int64_t)b * H_q + (int64_t)kvh * a.G + g) * D +
                    c16 * Geo::kCols;
          if constexpr (BF16) {
            uint32_t pk[Geo::kCols / 2];
#pragma unroll
            for (int c = 0; c < Geo::kCols / 2; ++c)
              pk[c] = (uint32_t)f32_to_bf16_rne(st.o[g][2 * c] * inv) |
                      ((uint32_t)f32_to_bf16_rne(st.o[g][2 * c + 1] * inv) << 16);
            if constexpr (Geo::kCols == 8) {
              *reinterpret_cast<u32x4_t*>(orow) = u32x4_t{pk[0], pk[1], pk[2], pk[3]};
            } else {
              *reinterpret_cast<uint2*>(orow) = uint2{pk[0], pk[1]};
            }
          } else {
#pragma unroll
            for (int c = 0; c < Geo::kCols; ++c) orow[c] = st.o[g][c] * inv;
          }
        }
      });
    } else if (item < a.cap_items) {
      const int64_t slot = ((int64_t)item * a.H_kv + kvh) * a.G;
      static_for<0, GP>([&](auto gi) {
        constexpr int g = decltype(gi)::value;
        if (g < a.G && (g & 3) == jr) {
          float* orow = a.ws_o + (slot + g) * D + c16 * Geo::kCols;
#pragma unroll
          for (int c = 0; c < Geo::kCols; ++c) orow[c] = st.o[g][c];
        }
      });
      if (lane < a.G) a.ws_ml[slot + lane] = make_float2(M, lt);
    }
  }
}

// Merges the split partials of one (sequence, KV head): 4 waves, wave w
// handles heads w, w+4, ...; lanes cover the head dimension.
template <bool BF16, int D>
__global__ void __launch_bounds__(256)
decode_merge_kernel(DecodeArgs a) {
  using T = std::conditional_t<BF16, uint16_t, float>;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int b = blockIdx.x / a.H_kv, kvh = blockIdx.x - (blockIdx.x / a.H_kv) * a.H_kv;
  const int32_t len_cap = a.max_blocks << a.log2_bs;
  const Plan plan = make_plan(a.lens, a.B, len_cap, a.target, lane);
  const int32_t L = clamp_len(a.lens, b, len_cap);
  const int32_t nsplit = (L + plan.part - 1) / plan.part;
  if (nsplit == 1) return;
  const int32_t H_q = a.H_kv * a.G;
  constexpr int kPer = D / kWave;
  if (nsplit == 0) {
    for (int g = wave; g < a.G; g += 4) {
      T* orow = reinterpret_cast<T*>(a.out) + ((int64_t)b * H_q + (int64_t)kvh * a.G + g) * D;
#pragma unroll
      for (int e = 0; e < kPer; ++e) orow[lane + e * kWave] = T(0);
    }
    return;
  }
  // First split index of sequence b.
  int32_t first = 0;
  for (int c = 0; c < b; c += kWave) {
    const int bb = c + lane;
    int32_t n = bb < b ? (clamp_len(a.lens, bb, len_cap) + plan.part - 1) / plan.part : 0;
    first += static_cast<int32_t>(wave_sum_i64(n));
  }
  if (first + nsplit > a.cap_items) return;
  for (int g = wave; g < a.G; g += 4) {
    float M = -3.0e38f;
    for (int s = lane; s < nsplit; s += kWave) {
      const int64_t slot = ((int64_t)(first + s) * a.H_kv + kvh) * a.G + g;
      M = fmaxf(M, a.ws_ml[slot].x);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    float acc[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) acc[e] = 0.f;
    float den = 0.f;
    for (int s = 0; s < nsplit; ++s) {
      const int64_t slot = ((int64_t)(first + s) * a.H_kv + kvh) * a.G + g;
      const float2 ml = a.ws_ml[slot];
      const float f = exp2f(ml.x - M);
      den = fmaf(f, ml.y, den);
      const float* orow = a.ws_o + slot * D;
#pragma unroll
      for (int e = 0; e < kPer; ++e) acc[e] = fmaf(f, orow[lane + e * kWave], acc[e]);
    }
    const float inv = 1.f / den;
    T* orow = reinterpret_cast<T*>(a.out) + ((int64_t)b * H_q + (int64_t)kvh * a.G + g) * D;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const float v = acc[e] * inv;
      if constexpr (BF16) {
        orow[lane + e * kWave] = f32_to_bf16_rne(v);
      } else {
        orow[lane + e * kWave] = v;
      }
    }
  }
}

// ----------------------------------------------------------- host helpers
constexpr int kDefaultItems = 2048;  // (split, KV head) items the plan aims at
constexpr int kMaxSplitGrid = 16384;

// Tuning override (read on every call): PA_DECODE_ITEMS = total number of
// (split, KV head) items the plan aims at.  Any value gives the same result
// up to fp32 rounding order.
int items_target_total() {
  const char* e = std::getenv("PA_DECODE_ITEMS");
  const int x = e ? std::atoi(e) : kDefaultItems;
  return x >= 1 && x <= (1 << 20) ? x : kDefaultItems;
}

int32_t target_per_head(int32_t H_kv) {
  const int32_t t = items_target_total() / H_kv;
  return t < 1 ? 1 : t;
}

int ilog2_exact(int32_t x) {
  if (x < 1 || (x & (x - 1))) return -1;
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

int elem_bytes(pa_dtype d) { return d == PA_BF16 ? 2 : 4; }

pa_status check_desc(const pa_cache_desc* desc) {
  if (!desc) return pa::fail(PA_ERR_INVALID_ARGUMENT, "desc is NULL");
  if (desc->num_blocks < 1 || desc->num_kv_heads < 1)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "num_blocks %d / num_kv_heads %d must be >= 1",
                    desc->num_blocks, desc->num_kv_heads);
  const int lg = ilog2_exact(desc->block_size);
  if (lg < 0 || lg > 8)
    return pa::fail(PA_ERR_UNSUPPORTED, "block_size %d is not a power of two in [1, 256]",
                    desc->block_size);
  if (desc->head_dim != 64 && desc->head_dim != 128)
    return pa::fail(PA_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", desc->head_dim);
  if (desc->dtype != PA_F32 && desc->dtype != PA_BF16)
    return pa::fail(PA_ERR_UNSUPPORTED, "dtype %d not in {PA_F32, PA_BF16}", desc->dtype);
  return PA_OK;
}

pa_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pa::fail(PA_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
  return PA_OK;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct WorkspaceLayout {
  size_t o_bytes, ml_off, total;
  int32_t cap_items;
};

WorkspaceLayout workspace_layout(const pa_cache_desc* d, int32_t B, int32_t H_q) {
  WorkspaceLayout w;
  w.cap_items = target_per_head(d->num_kv_heads) + B;
  w.o_bytes = align_up((size_t)w.cap_items * H_q * d->head_dim * sizeof(float), 256);
  w.ml_off = w.o_bytes;
  w.total = w.o_bytes + align_up((size_t)w.cap_items * H_q * sizeof(float2), 256);
  return w;
}

template <bool BF16, int D, int GP>
void launch_decode(const DecodeArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((decode_split_kernel<BF16, D, GP>), dim3(grid), dim3(kWave), 0, s, a);
  hipLaunchKernelGGL((decode_merge_kernel<BF16, D>), dim3(a.B * a.H_kv), dim3(256), 0, s, a);
}

template <bool BF16, int D>
void dispatch_g(const DecodeArgs& a, int grid, hipStream_t s) {
  if (a.G <= 1) launch_decode<BF16, D, 1>(a, grid, s);
  else if (a.G <= 2) launch_decode<BF16, D, 2>(a, grid, s);
  else if (a.G <= 4) launch_decode<BF16, D, 4>(a, grid, s);
  else if (a.G <= 8) launch_decode<BF16, D, 8>(a, grid, s);
  else launch_decode<BF16, D, 16>(a, grid, s);
}

}  // namespace

extern "C" {

pa_status pa_supported(const pa_cache_desc* desc, int32_t num_q_heads) {
  pa_status st = check_desc(desc);
  if (st != PA_OK) return st;
  if (num_q_heads < 1 || num_q_heads % desc->num_kv_heads)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "num_q_heads %d is not a multiple of %d",
                    num_q_heads, desc->num_kv_heads);
  const int32_t G = num_q_heads / desc->num_kv_heads;
  if (G > 16) return pa::fail(PA_ERR_UNSUPPORTED, "group size %d > 16", G);
  return PA_OK;
}

pa_status pa_cache_append(const void* k, const void* v, const int64_t* slot_mapping,
                          int32_t num_tokens, void* k_cache, void* v_cache,
                          const pa_cache_desc* desc, void* stream) {
  pa_status st = check_desc(desc);
  if (st != PA_OK) return st;
  if (num_tokens < 0) return pa::fail(PA_ERR_INVALID_ARGUMENT, "num_tokens %d < 0", num_tokens);
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "NULL pointer");
  const int32_t row_vecs = desc->head_dim * elem_bytes(desc->dtype) / 16;
  hipLaunchKernelGGL(cache_append_kernel, dim3(num_tokens), dim3(256), 0, (hipStream_t)stream,
                     (const uint4*)k, (const uint4*)v, slot_mapping, (uint4*)k_cache,
                     (uint4*)v_cache, (int64_t)desc->num_blocks * desc->block_size,
                     desc->block_size, desc->num_kv_heads, row_vecs);
  return check_launch("pa_cache_append");
}

pa_status pa_copy_blocks(const int32_t* src_dst_pairs, int32_t num_pairs, void* k_cache,
                         void* v_cache, const pa_cache_desc* desc, void* stream) {
  pa_status st = check_desc(desc);
  if (st != PA_OK) return st;
  if (num_pairs < 0) return pa::fail(PA_ERR_INVALID_ARGUMENT, "num_pairs %d < 0", num_pairs);
  if (num_pairs == 0) return PA_OK;
  if (!src_dst_pairs || !k_cache || !v_cache)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (num_pairs > desc->num_blocks)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "num_pairs %d > num_blocks %d", num_pairs,
                    desc->num_blocks);
  const int64_t block_vecs = (int64_t)desc->num_kv_heads * desc->block_size * desc->head_dim *
                             elem_bytes(desc->dtype) / 16;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs, 2), dim3(256), 0, (hipStream_t)stream,
                     src_dst_pairs, (uint4*)k_cache, (uint4*)v_cache, desc->num_blocks,
                     block_vecs);
  return check_launch("pa_copy_blocks");
}

pa_status pa_decode_workspace_size(const pa_cache_desc* desc, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t max_blocks_per_seq,
                                   size_t* bytes) {
  pa_status st = pa_supported(desc, num_q_heads);
  if (st != PA_OK) return st;
  if (!bytes) return pa::fail(PA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (num_seqs < 0 || max_blocks_per_seq < 1)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "num_seqs %d / max_blocks_per_seq %d", num_seqs,
                    max_blocks_per_seq);
  *bytes = workspace_layout(desc, num_seqs, num_q_heads).total;
  return PA_OK;
}

pa_status pa_decode(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t num_seqs, int32_t block_size,
                    float scale, void* out, int32_t num_q_heads, const pa_cache_desc* desc,
                    void* workspace, size_t workspace_bytes, void* stream) {
  pa_status st = pa_supported(desc, num_q_heads);
  if (st != PA_OK) return st;
  if (block_size != desc->block_size)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "block_size %d != desc->block_size %d", block_size,
                    desc->block_size);
  if (num_seqs < 0 || max_blocks_per_seq < 1)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "num_seqs %d / max_blocks_per_seq %d", num_seqs,
                    max_blocks_per_seq);
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "max_blocks_per_seq * block_size overflows int32");
  if (!std::isfinite(scale)) return pa::fail(PA_ERR_INVALID_ARGUMENT, "scale is not finite");
  if (num_seqs == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out || !workspace)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
  const WorkspaceLayout wl = workspace_layout(desc, num_seqs, num_q_heads);
  if (workspace_bytes < wl.total)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "workspace %zu bytes < %zu needed", workspace_bytes,
                    wl.total);
  DecodeArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.tables = block_tables;
  a.lens = context_lens;
  a.out = out;
  a.ws_o = reinterpret_cast<float*>(workspace);
  a.ws_ml = reinterpret_cast<float2*>(reinterpret_cast<char*>(workspace) + wl.ml_off);
  a.B = num_seqs;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = desc->num_blocks;
  a.H_kv = desc->num_kv_heads;
  a.G = num_q_heads / desc->num_kv_heads;
  a.log2_bs = ilog2_exact(block_size);
  a.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  a.target = target_per_head(desc->num_kv_heads);
  a.cap_items = wl.cap_items;
  const int64_t grid64 = (int64_t)wl.cap_items * a.H_kv;
  const int grid = static_cast<int>(grid64 < kMaxSplitGrid ? grid64 : kMaxSplitGrid);
  hipStream_t s = (hipStream_t)stream;
  const bool bf16 = desc->dtype == PA_BF16;
  if (bf16 && desc->head_dim == 128) dispatch_g<true, 128>(a, grid, s);
  else if (bf16) dispatch_g<true, 64>(a, grid, s);
  else if (desc->head_dim == 128) dispatch_g<false, 128>(a, grid, s);
  else dispatch_g<false, 64>(a, grid, s);
  return check_launch("pa_decode");
}

}  // extern "C"
