// Single-query (decode) attention that reads K/V through per-sequence block
// tables (gfx950 / CDNA4, wave64).
//
// Sources: "Paged Attention" (klaylearn.com glossary), body: the kernel
// turns a token position into (logical block, offset), looks the physical
// block up in the sequence's table and reads K and V there without first
// gathering the sequence; "What is paged attention in vLLM, and why does it
// matter?" (interview.clozo.ai), Step 3: the attention kernel follows the
// table; "PagedAttention - AI Glossary" (modelrefs.com), Example: the
// attention arithmetic itself is unchanged by paging.
//
// Work decomposition:
//  * A segment is one (sequence b, KV head) pair; it has ceil(L_b / 16)
//    tiles of 16 tokens.  All tiles of all segments are numbered in one flat
//    order (b, KV head, tile).  Workgroup w takes the equal share
//    [T*w/W, T*(w+1)/W) of the T tiles and wave v of the workgroup the
//    equal contiguous part v of that share, so every wave streams the same
//    number of K/V bytes whatever the length mix.
//  * Context lengths are first copied into LDS with their prefix sums over
//    sequences, so all waves of a workgroup see one consistent snapshot.
//  * A wave walks its part as pieces, one per segment it meets; each piece
//    is a straight pipelined loop over its tiles (NBUF tiles of loads in
//    flight), with the segment's query rows and physical block ids fetched
//    before the loop.  A segment wholly inside the wave's part is written
//    out by the wave.  Other pieces leave their online-softmax state in LDS;
//    after one barrier the leading wave of each such segment merges the
//    states: into the output if the segment lies inside the workgroup's
//    share, else into a partial in the workspace.
//  * A second, small kernel merges the partials of segments cut by share
//    boundaries (the workgroup that holds a segment's first part leaves a
//    record for it), so no cross-workgroup synchronisation is needed.
//  * Per tile: the K rows of the 16 tokens are the A operand of one MFMA
//    chain (v_mfma_f32_16x16x32_bf16, or 16x16x4_f32 for fp32 pools) whose
//    B operand is the KV head's G query rows, loaded straight from memory
//    with 16-byte loads (lane l holds a 16-byte piece of token l % 16's
//    row).  The logits land in lane 16*j + g (head g, tokens 4j..4j+3); each
//    16-lane row keeps its own running max and sum.  P*V runs on the VALU in
//    fp32: lane 16*j + c owns D/16 output columns for the V rows of tokens
//    4j..4j+3, with the probabilities broadcast by DPP.
//  * Blocks of >= 16 tokens are read through a buffer resource spanning the
//    tile; the padding tiles of the pipeline get a zero-length resource, so
//    every loop iteration issues the same loads and each use waits only for
//    its own tile.
//  * Masked positions (past the context length) are removed by select, so
//    garbage or NaN in unused slots of a block cannot reach the output.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace {

using pa::bf16x8_t;
using pa::floatx4_t;
using pa::kWave;
using pa::u32x4_t;

constexpr int kTile = 16;         // tokens per tile (one MFMA row block)
constexpr int kMaxWGs = 1024;     // the workspace holds partials for this many workgroups
constexpr int kDefaultWGs = 256;  // one workgroup per compute unit
constexpr int kMaxSeqs = 8192;    // lengths snapshot in LDS
constexpr int kRecInts = 8;       // ints per cut-segment record
constexpr int kTaskHead = 4;      // ints before the contributor slots of a merge task
constexpr int kMergeWG = 256;     // threads of the partial-merge kernel
constexpr size_t kMaxLds = 160 * 1024;
#ifndef PA_DECODE_NB_BF16
#define PA_DECODE_NB_BF16 3  // tiles per batch for bf16 pools (build-time tuning knob)
#endif

struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* tables;
  const int32_t* lens;
  void* out;
  float* ws_o;       // [2 * kMaxWGs][G][D] unnormalised partial outputs
  float* ws_m;       // [2 * kMaxWGs][G] running max (log2 units)
  float* ws_l;       // [2 * kMaxWGs][G] sum of exp2(x - max)
  int32_t* records;  // [kMaxWGs][kRecInts] cut segment led by each workgroup
  int32_t B;
  int32_t max_blocks;
  int32_t num_blocks;
  int32_t H_kv;
  int32_t G;
  int32_t log2_bs;
  float scale_log2;  // scale * log2(e)
};

template <bool BF16, int D>
struct Geometry {
  static constexpr int kElem = BF16 ? 2 : 4;
  static constexpr int kRowBytes = D * kElem;
  static constexpr int kKPieces = kRowBytes / 64;     // 16-byte K pieces per lane per tile
  static constexpr int kVWords = kRowBytes / 16 / 4;  // 32-bit words of V per lane per token
  static constexpr int kCols = D / 16;                // output columns per lane
  static constexpr int kQRegs = BF16 ? kKPieces : 1;  // query as bf16 MFMA operand
  static constexpr int kQF32 = BF16 ? 1 : kKPieces * 4;
  static_assert(kRowBytes % 64 == 0, "row must be a multiple of 64 bytes");
};

template <bool BF16, int D>
struct TileRegs {
  using Geo = Geometry<BF16, D>;
  u32x4_t k[Geo::kKPieces];
  uint32_t v[4][Geo::kVWords];
};

template <bool BF16, int D, int GP>
struct WaveState {
  using Geo = Geometry<BF16, D>;
  float m;                  // lane 16j+g: running max of head g over row j (log2 units)
  float l;                  // lane 16j+g: running sum of exp2(x - m)
  float o[GP][Geo::kCols];  // lane 16j+c: unnormalised output, columns of chunk c

  __device__ __forceinline__ void reset() {
    m = -3.0e38f;
    l = 0.f;
#pragma unroll
    for (int g = 0; g < GP; ++g)
#pragma unroll
      for (int c = 0; c < Geo::kCols; ++c) o[g][c] = 0.f;
  }
};

__device__ __forceinline__ int32_t uni(int32_t x) { return __builtin_amdgcn_readfirstlane(x); }

// One segment (sequence b, KV head kvh) and its flat tile range [S0, S1).
struct Seg {
  int32_t b, kvh, nt, L, S0, S1;
};

// Largest b in [0, B) with PB[b] * H_kv <= f (PB: exclusive prefix sums of
// tiles per sequence, in LDS).
__device__ __forceinline__ int32_t find_seq(const int32_t* PB, int32_t B, int32_t H_kv,
                                            int32_t f) {
  int32_t lo = 0, hi = B - 1;
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if (PB[mid] * H_kv <= f) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// The segment holding flat tile f (0 <= f < total); f is wave-uniform.
__device__ __forceinline__ Seg seg_containing(const int32_t* PB, const int32_t* Ls, int32_t B,
                                              int32_t H_kv, int32_t f) {
  Seg s;
  s.b = uni(find_seq(PB, B, H_kv, f));
  const int32_t pb = uni(PB[s.b]);
  s.nt = uni(PB[s.b + 1]) - pb;
  s.kvh = (f - pb * H_kv) / s.nt;
  s.S0 = pb * H_kv + s.kvh * s.nt;
  s.S1 = s.S0 + s.nt;
  s.L = uni(Ls[s.b]);
  return s;
}

// Moves s to the next non-empty segment in flat order.  Called only while
// one exists; should the snapshot say otherwise, s becomes an empty segment
// at the end of every range, which stops every loop that walks segments.
__device__ __forceinline__ void seg_advance(Seg& s, const int32_t* PB, const int32_t* Ls,
                                            int32_t B, int32_t H_kv) {
  if (s.kvh + 1 < H_kv) {
    s.kvh += 1;
    s.S0 = s.S1;
    s.S1 += s.nt;
    return;
  }
  int32_t b = s.b + 1;
  while (b < B && uni(PB[b + 1]) == uni(PB[b])) ++b;
  if (b >= B) {
    s.S0 = s.S1 = 0x7FFFFFFF;
    return;
  }
  s.b = b;
  s.kvh = 0;
  s.S0 = uni(PB[b]) * H_kv;
  s.nt = uni(PB[b + 1]) - uni(PB[b]);
  s.S1 = s.S0 + s.nt;
  s.L = uni(Ls[b]);
}

// A wave-uniform pointer, moved to SGPRs.
__device__ __forceinline__ char* uniform_ptr(const char* p) {
  const uint64_t x = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x >> 32));
  return reinterpret_cast<char*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Buffer-resource word 3 for raw dword loads on gfx9-family parts (32-bit
// data format; a zero format would make every load return zero).
constexpr int32_t kRsrcWord3 = 0x00020000;

// Issues the K/V loads of tile t of a segment (KV head kvh) whose 16 rows
// lie in physical block `phys` (blocks of >= 16 tokens).  The rows are read
// through a buffer resource spanning exactly them; pipeline padding
// (`valid` false) gets a zero-length resource, so its loads return zeros
// without touching memory.  Rows past the context length stay inside the
// block and are masked when consumed.
template <bool BF16, int D>
__device__ __forceinline__ void issue_tile(TileRegs<BF16, D>& r, const DecodeArgs& a,
                                           int32_t phys, int32_t t, int32_t kvh, int lane,
                                           bool valid) {
  using Geo = Geometry<BF16, D>;
  const int bs_log = a.log2_bs;
  const int32_t bs = 1 << bs_log;
  const int jr = lane >> 4, c16 = lane & 15;
  phys = min(max(phys, 0), a.num_blocks - 1);
  const int64_t off0 =
      (((int64_t)phys * a.H_kv + kvh) * bs + ((t * kTile) & (bs - 1))) * Geo::kRowBytes;
  // The resource must live in SGPRs: every input is wave-uniform, and
  // readfirstlane says so to the compiler (otherwise it wraps each load in
  // a loop over the distinct values of the resource).
  const int32_t nrec = uni(valid ? kTile * Geo::kRowBytes : 0);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr(reinterpret_cast<const char*>(a.k_cache) + off0), 0, nrec, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr(reinterpret_cast<const char*>(a.v_cache) + off0), 0, nrec, kRsrcWord3);
  const int32_t ko = (lane & 15) * Geo::kRowBytes + jr * 16;
#pragma unroll
  for (int p = 0; p < Geo::kKPieces; ++p)
    r.k[p] = __builtin_bit_cast(u32x4_t,
                                __builtin_amdgcn_raw_buffer_load_b128(rk, ko + p * 64, 0, 0));
  const int32_t vo = (jr * 4) * Geo::kRowBytes + c16 * (Geo::kVWords * 4);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int h = 0; h < Geo::kVWords; h += 4) {
      if constexpr (Geo::kVWords >= 4) {
        const u32x4_t x = __builtin_bit_cast(
            u32x4_t,
            __builtin_amdgcn_raw_buffer_load_b128(rv, vo + q * Geo::kRowBytes + h * 4, 0, 0));
        r.v[q][h + 0] = x[0];
        r.v[q][h + 1] = x[1];
        r.v[q][h + 2] = x[2];
        r.v[q][h + 3] = x[3];
      } else {
        const uint2 x = __builtin_bit_cast(
            uint2, __builtin_amdgcn_raw_buffer_load_b64(rv, vo + q * Geo::kRowBytes, 0, 0));
        r.v[q][0] = x.x;
        r.v[q][1] = x.y;
      }
    }
  }
}

// Same for blocks of fewer than 16 tokens: a tile spans nbt = 16 / bs
// blocks, whose ids are lanes jl*nbt .. jl*nbt + nbt - 1 of phys_v; every
// lane reads its own rows' blocks.  Rows past the context length L (and
// padding tiles, whose index the caller clamps) read the last valid token
// again.
template <bool BF16, int D>
__device__ __forceinline__ void issue_tile_small(TileRegs<BF16, D>& r, const DecodeArgs& a,
                                                 int32_t phys_v, int32_t jl, int32_t t,
                                                 int32_t kvh, int32_t L, int nbt, int lane) {
  using Geo = Geometry<BF16, D>;
  const int bs_log = a.log2_bs;
  const int32_t bs = 1 << bs_log;
  const int jr = lane >> 4, c16 = lane & 15;
  const int32_t src = jl * nbt;
  const int32_t t0 = t * kTile;
  auto row_addr = [&](int32_t row, const void* base) -> const char* {
    const int32_t tok = min(t0 + row, L - 1);
    const int32_t sub = (tok - t0) >> bs_log;
    const int32_t phys = min(max(__shfl(phys_v, src + sub), 0), a.num_blocks - 1);
    return reinterpret_cast<const char*>(base) +
           (((int64_t)phys * a.H_kv + kvh) * bs + (tok & (bs - 1))) * Geo::kRowBytes;
  };
  const char* kp = row_addr(lane & 15, a.k_cache) + jr * 16;
#pragma unroll
  for (int p = 0; p < Geo::kKPieces; ++p) r.k[p] = *reinterpret_cast<const u32x4_t*>(kp + p * 64);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const char* vp = row_addr(jr * 4 + q, a.v_cache) + c16 * (Geo::kVWords * 4);
#pragma unroll
    for (int h = 0; h < Geo::kVWords; h += 4) {
      if constexpr (Geo::kVWords >= 4) {
        u32x4_t x = *reinterpret_cast<const u32x4_t*>(vp + h * 4);
        r.v[q][h + 0] = x[0];
        r.v[q][h + 1] = x[1];
        r.v[q][h + 2] = x[2];
        r.v[q][h + 3] = x[3];
      } else {
        uint2 x = *reinterpret_cast<const uint2*>(vp);
        r.v[q][0] = x.x;
        r.v[q][1] = x.y;
      }
    }
  }
}

// Consumes one tile: logits by MFMA, online softmax per 16-lane row, P*V.
// t0 = first token of the tile within its sequence, end = context length.
template <bool BF16, int D, int GP>
__device__ __forceinline__ void consume_tile(WaveState<BF16, D, GP>& st,
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
        s = __builtin_amdgcn_mfma_f32_16x16x4f32(pa::as_float(r.k[p][e]), qf32[4 * p + e], s, 0,
                                                 0, 0);
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

  // V rows of this lane's 4 tokens widened to fp32; masked rows are zeroed
  // by select so that garbage (even NaN) in unused slots cannot leak in.
  float vf[4][Geo::kCols];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bool ok = !tail || (t0 + jr * 4 + q < end);
#pragma unroll
    for (int w = 0; w < Geo::kVWords; ++w) {
      if constexpr (BF16) {
        vf[q][2 * w] = ok ? pa::bf16_lo(r.v[q][w]) : 0.f;
        vf[q][2 * w + 1] = ok ? pa::bf16_hi(r.v[q][w]) : 0.f;
      } else {
        vf[q][w] = ok ? pa::as_float(r.v[q][w]) : 0.f;
      }
    }
  }
  pa::static_for<0, GP>([&](auto gi) {
    constexpr int g = decltype(gi)::value;
    const float al = pa::row_bcast<g>(alpha);
    float p[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) p[q] = pa::row_bcast<g>(pr[q]);
#pragma unroll
    for (int c = 0; c < Geo::kCols; ++c) {
      float acc = st.o[g][c] * al;
#pragma unroll
      for (int q = 0; q < 4; ++q) acc = fmaf(p[q], vf[q][c], acc);
      st.o[g][c] = acc;
    }
  });
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Per-wave state over one piece, bf16 pools (P*V by MFMA).
//  ref: lane 16j + g: reference max of head g (log2 units), equal in all rows.
//  l:   lane 16j + g: sum of the (bf16-rounded) weights of head g over the
//       tokens of row j.
//  acc[blk]: lane 16j + c, register r: unnormalised output of head 4j + r at
//       column (D/16)*c + blk.
template <int D>
struct MfmaState {
  static constexpr int kBlk = D / 16;
  float ref;
  float l;
  floatx4_t acc[kBlk];

  __device__ __forceinline__ void reset() {
    ref = -3.0e38f;
    l = 0.f;
#pragma unroll
    for (int b = 0; b < kBlk; ++b) acc[b] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  }
};

// Consumes one tile (bf16): logits S = K q^T by MFMA (lane 16j + g holds
// heads g, tokens 4j..4j+3); weights p = 2^(x - ref) against a reference
// max that is raised (and the accumulators rescaled) only when a logit
// exceeds it by more than 2^8, so the common tile needs no cross-lane
// reduction; then O += P V by MFMA with P (heads x tokens) exactly where the
// logits are and V (tokens x columns) made from the lane's own V rows.
// Weights past the context length (or for heads >= G) are zero, and so are
// V rows past the context length, so garbage in unused slots cannot leak.
template <int D>
__device__ __forceinline__ void consume_tile_mfma(MfmaState<D>& st,
                                                  const TileRegs<true, D>& r,
                                                  const u32x4_t* qf, float scale_log2,
                                                  int32_t t0, int32_t end, int32_t G, int lane) {
  using Geo = Geometry<true, D>;
  constexpr int kBlk = MfmaState<D>::kBlk;
  const int jr = lane >> 4, c16 = lane & 15;
  floatx4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < Geo::kKPieces; ++p)
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, r.k[p]),
                                                __builtin_bit_cast(bf16x8_t, qf[p]), s, 0, 0, 0);
  const bool tail = t0 + kTile > end;  // uniform
  const bool live = c16 < G;
  float x[4];
  bool hi = false;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    x[q] = s[q] * scale_log2;
    if (!live || t0 + jr * 4 + q >= end) x[q] = -INFINITY;
    hi = hi || x[q] > st.ref + 8.f;
  }
  if (__ballot(hi) != 0) {  // uniform: raise the reference
    float mt = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float nref = fmaxf(st.ref, mt);
    const float f = __builtin_amdgcn_exp2f(st.ref - nref);
    st.l *= f;
    st.ref = nref;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float fr = __shfl(f, 4 * jr + q);  // head 4j + q
#pragma unroll
      for (int b = 0; b < kBlk; ++b) st.acc[b][q] *= fr;
    }
  }
  const f32x2_t p01 = {__builtin_amdgcn_exp2f(x[0] - st.ref), __builtin_amdgcn_exp2f(x[1] - st.ref)};
  const f32x2_t p23 = {__builtin_amdgcn_exp2f(x[2] - st.ref), __builtin_amdgcn_exp2f(x[3] - st.ref)};
  const uint32_t a01 = __builtin_bit_cast(uint32_t, __builtin_convertvector(p01, bf16x2_t));
  const uint32_t a23 = __builtin_bit_cast(uint32_t, __builtin_convertvector(p23, bf16x2_t));
  st.l += (pa::bf16_lo(a01) + pa::bf16_hi(a01)) + (pa::bf16_lo(a23) + pa::bf16_hi(a23));
  const s16x4_t pa_ = __builtin_bit_cast(s16x4_t, (uint64_t)a01 | ((uint64_t)a23 << 32));
  uint32_t m01 = 0xFFFFFFFFu, m23 = 0xFFFFFFFFu;
  if (tail) {
    const int32_t row0 = t0 + jr * 4;
    m01 = (row0 + 0 < end ? 0x0000FFFFu : 0u) | (row0 + 1 < end ? 0xFFFF0000u : 0u);
    m23 = (row0 + 2 < end ? 0x0000FFFFu : 0u) | (row0 + 3 < end ? 0xFFFF0000u : 0u);
  }
#pragma unroll
  for (int b = 0; b < kBlk; ++b) {
    const int w = b >> 1;
    const uint32_t sel = (b & 1) ? 0x07060302u : 0x05040100u;
    const uint32_t v01 = __builtin_amdgcn_perm(r.v[1][w], r.v[0][w], sel) & m01;
    const uint32_t v23 = __builtin_amdgcn_perm(r.v[3][w], r.v[2][w], sel) & m23;
    const s16x4_t vb = __builtin_bit_cast(s16x4_t, (uint64_t)v01 | ((uint64_t)v23 << 32));
    st.acc[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa_, vb, st.acc[b], 0, 0, 0);
  }
}

// Loads the G query rows of segment (b, kvh) as the MFMA B operand (lane
// 16j + g holds 16-byte pieces of head g; zero for g >= G).
template <bool BF16, int D>
__device__ __forceinline__ void load_q(const DecodeArgs& a, int32_t b, int32_t kvh, u32x4_t* qf,
                                       float* qf32, int lane) {
  using Geo = Geometry<BF16, D>;
  const int jr = lane >> 4, c16 = lane & 15;
  const bool live = c16 < a.G;
  const int64_t row = ((int64_t)b * a.H_kv + kvh) * a.G + (live ? c16 : 0);
  const char* qb = reinterpret_cast<const char*>(a.q) + row * Geo::kRowBytes + jr * 16;
#pragma unroll
  for (int p = 0; p < Geo::kKPieces; ++p) {
    u32x4_t x = *reinterpret_cast<const u32x4_t*>(qb + p * 64);
    if (!live) x = u32x4_t{0, 0, 0, 0};
    if constexpr (BF16) {
      qf[p] = x;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) qf32[4 * p + e] = pa::as_float(x[e]);
    }
  }
}

// Adds n >= 1 softmax partials (max m_i, sum l_i, unnormalised o_i of one
// output element) by the rescaled-sum rule; `get(i, m, o, l)` fetches
// partial i.  Partials are fetched kBatch at a time with indices clamped to
// n - 1 (the extra copies get weight zero), so each batch's loads are issued
// together, one round trip per batch.
struct Merged {
  float mx, acc, den;  // max, unnormalised output, sum; the result is acc / den
};

template <int kBatch, typename Get>
__device__ __forceinline__ Merged merge_partials(int32_t n, Get&& get) {
  float mx = -3.0e38f, acc = 0.f, den = 0.f;
  for (int32_t i0 = 0; i0 < n; i0 += kBatch) {
    float pm[kBatch], po[kBatch], pl[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) get(min(i0 + k, n - 1), pm[k], po[k], pl[k]);
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
      if (i0 + k >= n) pm[k] = -3.0e38f;
    float cm = mx;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) cm = fmaxf(cm, pm[k]);
    const float r = __builtin_amdgcn_exp2f(mx - cm);
    acc *= r;
    den *= r;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const float f = i0 + k < n ? __builtin_amdgcn_exp2f(pm[k] - cm) : 0.f;
      acc = fmaf(f, po[k], acc);
      den = fmaf(f, pl[k], den);
    }
    mx = cm;
  }
  return Merged{mx, acc, den};
}

// Largest w with floor(T * w / W) <= f: the share (of W equal shares of T
// units) that holds unit f, for 0 <= f < T.
__device__ __forceinline__ int32_t share_of(int32_t f, int32_t T, int32_t W) {
  return static_cast<int32_t>((((int64_t)f + 1) * W - 1) / T);
}

template <bool BF16>
__device__ __forceinline__ void store_out(void* out, int64_t i, float x) {
  if constexpr (BF16) reinterpret_cast<uint16_t*>(out)[i] = pa::f32_to_bf16_rne(x);
  else reinterpret_cast<float*>(out)[i] = x;
}

template <bool BF16, int D, int GP, int kNW, int NBUF, bool kSmall>
__global__ void __launch_bounds__(kNW * kWave)
decode_kernel(DecodeArgs a) {
  using Geo = Geometry<BF16, D>;
  constexpr int kWG = kNW * kWave;
  constexpr int kTaskInts = kTaskHead + kNW;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), v = tid >> 6;
  const int jr = lane >> 4, c16 = lane & 15;
  const int32_t wg = blockIdx.x, nwg = gridDim.x;
  const int32_t B = a.B, H_kv = a.H_kv, G = a.G, H_q = H_kv * G;

  // LDS: per wave two parked states (o[G][D], m[G], l[G]), then the lengths.
  const int32_t slot_floats = G * D + 2 * G;
  float* lds_st = reinterpret_cast<float*>(smem);                       // [kNW][2][slot]
  int32_t* PB = reinterpret_cast<int32_t*>(lds_st + kNW * 2 * slot_floats);  // [B + 1]
  int32_t* Ls = PB + B + 1;                                            // [B]
  int32_t* misc = Ls + B;                                              // [kNW]
  int32_t* tasks = misc + kNW;                                         // [2 * kNW][kTaskInts]

  // ---- lengths snapshot and prefix sums of tiles per sequence
  const int32_t len_cap = a.max_blocks << a.log2_bs;
  int32_t carry = 0;
  for (int32_t c = 0; c < B; c += kWG) {
    const int32_t b = c + tid;
    int32_t L = 0;
    if (b < B) {
      L = a.lens[b];
      L = L < 0 ? 0 : (L > len_cap ? len_cap : L);
      Ls[b] = L;
    }
    const int32_t nt = (L + kTile - 1) / kTile;
    const int32_t incl = pa::wave_incl_scan(nt, lane);
    if (lane == kWave - 1) misc[v] = incl;
    __syncthreads();
    int32_t pre = carry, tot = 0;
#pragma unroll
    for (int u = 0; u < kNW; ++u) {
      const int32_t x = misc[u];
      pre += u < v ? x : 0;
      tot += x;
    }
    if (b < B) PB[b] = pre + incl - nt;
    carry += tot;
    __syncthreads();
  }
  if (tid == 0) PB[B] = carry;
  __syncthreads();

  const int32_t Tt = uni(PB[B]) * H_kv;  // flat tiles (host bounds it below 2^31)
  const int32_t F0 = static_cast<int32_t>((int64_t)Tt * wg / nwg);
  const int32_t F1 = static_cast<int32_t>((int64_t)Tt * (wg + 1) / nwg);
  int32_t* rec = a.records + wg * kRecInts;

  // Sequences with no context get a zero row (workgroup b % W writes it).
  for (int32_t b = wg; b < B; b += nwg) {
    if (Ls[b] == 0) {
      for (int32_t e = tid; e < H_q * D; e += kWG)
        store_out<BF16>(a.out, (int64_t)b * H_q * D + e, 0.f);
    }
  }
  if (F0 >= F1) {
    if (tid == 0) rec[0] = 0;
    return;
  }

  // ---- this wave's contiguous part [G0, G1) of the share
  const int32_t span = F1 - F0;
  auto part_start = [&](int32_t w) { return F0 + static_cast<int32_t>((int64_t)span * w / kNW); };
  const int32_t G0 = part_start(v), G1 = part_start(v + 1);
  const int log2_bs = a.log2_bs;
  const int nbt = log2_bs >= 4 ? 1 : (kTile >> log2_bs);  // table lanes per tile
  const int tpc_log = log2_bs >= 4 ? 6 : 2 + log2_bs;       // log2(tiles per table chunk)
  auto slot_ptr = [&](int w, int k) { return lds_st + (w * 2 + k) * slot_floats; };

  if (G0 < G1) {
    Seg s = seg_containing(PB, Ls, B, H_kv, G0);
    while (true) {
      // ---- one piece: tiles [t0, t0 + n) of segment s
      const int32_t t0 = max(s.S0, G0) - s.S0;
      const int32_t n = min(s.S1, G1) - s.S0 - t0;
      u32x4_t qf[Geo::kQRegs];
      float qf32[Geo::kQF32];
      load_q<BF16, D>(a, s.b, s.kvh, qf, qf32, lane);
      // The loop body has no branches: padding steps past the piece's
      // last tile issue zero-length loads and consume a fully masked tile
      // (a no-op on the state), so every use waits only for its own loads.
      std::conditional_t<BF16, MfmaState<D>, WaveState<false, D, GP>> st;
      st.reset();
      TileRegs<BF16, D> buf[NBUF];
      auto consume = [&](const TileRegs<BF16, D>& r, int32_t j) {
        const int32_t tok0 = kTile * (t0 + j);
        const int32_t end = j < n ? s.L : tok0;  // padding: every row masked
        if constexpr (BF16) consume_tile_mfma<D>(st, r, qf, a.scale_log2, tok0, end, G, lane);
        else consume_tile(st, r, qf, qf32, a.scale_log2, tok0, end, lane);
      };
      if constexpr (!kSmall) {
        // Physical block ids by scalar loads (the table is read-only during
        // the kernel), one tile ahead of their use.
        const int32_t __attribute__((address_space(4)))* trow =
            (const int32_t __attribute__((address_space(4)))*)uniform_ptr(
                reinterpret_cast<const char*>(a.tables + (int64_t)s.b * a.max_blocks));
        auto phys_of = [&](int32_t j) -> int32_t {
          return trow[uni(((t0 + min(j, n - 1)) * kTile) >> log2_bs)];
        };
        // Batches: each iteration issues the loads of NBUF tiles, then
        // consumes them, so no load is in flight across the loop's back edge
        // (the other waves of the SIMD cover the gap between batches).
        for (int32_t j0 = 0; j0 < n; j0 += NBUF) {
          int32_t ph[NBUF];
#pragma unroll
          for (int u = 0; u < NBUF; ++u) ph[u] = phys_of(j0 + u);
#pragma unroll
          for (int u = 0; u < NBUF; ++u)
            issue_tile<BF16, D>(buf[u], a, ph[u], t0 + min(j0 + u, n - 1), s.kvh, lane,
                                j0 + u < n);
          // Keep every load of the batch ahead of the first use: left alone,
          // the scheduler sinks loads next to their uses to save registers.
          __builtin_amdgcn_sched_barrier(0);
          pa::static_for<0, NBUF>([&](auto U) { consume(buf[decltype(U)::value], j0 + decltype(U)::value); });
        }
      } else {
        // Blocks smaller than a tile: block ids of a chunk of tiles in a
        // VGPR (one per lane), one chunk ahead.  Lanes past the piece repeat
        // its last tile, so the gather is unconditional.
        const int32_t* trow = a.tables + (int64_t)s.b * a.max_blocks;
        auto describe = [&](int32_t chunk) -> int32_t {
          const int32_t i = min((chunk << tpc_log) + lane / nbt, n - 1);
          const int32_t tok = min((t0 + i) * kTile + ((lane & (nbt - 1)) << log2_bs), s.L - 1);
          return trow[tok >> log2_bs];
        };
        int32_t dA = describe(0), dB = describe(1);
        int32_t chunkA = 0;
        auto issue = [&](TileRegs<BF16, D>& r, int32_t j) {
          const int32_t jj = min(j, n - 1);
          const int32_t c = jj >> tpc_log;
          if (c != chunkA) {
            dA = dB;
            chunkA = c;
            dB = describe(c + 1);
          }
          issue_tile_small<BF16, D>(r, a, dA, jj - (c << tpc_log), t0 + jj, s.kvh, s.L, nbt,
                                    lane);
        };
        pa::static_for<0, NBUF - 1>([&](auto U) { issue(buf[decltype(U)::value], decltype(U)::value); });
        for (int32_t j0 = 0; j0 < n; j0 += NBUF) {
          pa::static_for<0, NBUF>([&](auto U) {
            constexpr int u = decltype(U)::value;
            const int32_t j = j0 + u;
            issue(buf[(u + NBUF - 1) % NBUF], j + NBUF - 1);
            consume(buf[u], j);
          });
        }
      }

      const bool whole = s.S0 >= G0 && s.S1 <= G1;
      float* slot = slot_ptr(v, s.S0 < G0 ? 0 : 1);
      if constexpr (BF16) {
        // ---- finish the piece: sums over the 4 rows; the accumulators
        // already hold whole tiles (lane 16j + c, register r: head 4j + r).
        constexpr int kBlk = D / 16;
        float lt = st.l;
        lt += __shfl_xor(lt, 16);
        lt += __shfl_xor(lt, 32);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int g = 4 * jr + q;
          const float lg = __shfl(lt, g);  // lane g holds head g's sum
          if (g < G) {
            if (whole) {
              const float inv = 1.f / lg;
              uint32_t wv[kBlk / 2];
#pragma unroll
              for (int i = 0; i < kBlk / 2; ++i) {
                const f32x2_t pr = {st.acc[2 * i][q] * inv, st.acc[2 * i + 1][q] * inv};
                wv[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2_t));
              }
              char* dst = reinterpret_cast<char*>(a.out) +
                          ((((int64_t)s.b * H_kv + s.kvh) * G + g) * D + kBlk * c16) * 2;
              if constexpr (kBlk == 8) *reinterpret_cast<u32x4_t*>(dst) = u32x4_t{wv[0], wv[1], wv[2], wv[3]};
              else *reinterpret_cast<uint2*>(dst) = uint2{wv[0], wv[1]};
            } else {
              float* dst = slot + g * D + kBlk * c16;
#pragma unroll
              for (int i = 0; i < kBlk; ++i) dst[i] = st.acc[i][q];
            }
          }
        }
        if (!whole && lane < G) {
          slot[G * D + lane] = st.ref;
          slot[G * D + G + lane] = lt;
        }
      } else {
      // ---- merge the 4 row states (lanes g, 16+g, 32+g, 48+g hold head g)
        float M = fmaxf(st.m, __shfl_xor(st.m, 16));
        M = fmaxf(M, __shfl_xor(M, 32));
        const float sc = exp2f(st.m - M);
        float lt = st.l * sc;
        lt += __shfl_xor(lt, 16);
        lt += __shfl_xor(lt, 32);
        pa::static_for<0, GP>([&](auto gi) {
          constexpr int g = decltype(gi)::value;
          const float f = pa::row_bcast<g>(sc);
          const float inv = 1.f / pa::row_bcast<g>(lt);
          float o[Geo::kCols];
#pragma unroll
          for (int c = 0; c < Geo::kCols; ++c) {
            o[c] = st.o[g][c] * f;
            o[c] += __shfl_xor(o[c], 16);
            o[c] += __shfl_xor(o[c], 32);
          }
          if (g < G && (g & 3) == jr) {
            if (whole) {
              const int64_t base = (((int64_t)s.b * H_kv + s.kvh) * G + g) * D + c16 * Geo::kCols;
#pragma unroll
              for (int c = 0; c < Geo::kCols; ++c) store_out<BF16>(a.out, base + c, o[c] * inv);
            } else {
#pragma unroll
              for (int c = 0; c < Geo::kCols; ++c) slot[g * D + c16 * Geo::kCols + c] = o[c];
            }
          }
        });
        if (!whole && lane < G) {
          slot[G * D + lane] = M;
          slot[G * D + G + lane] = lt;
        }
      }
      if (s.S1 >= G1) break;
      seg_advance(s, PB, Ls, B, H_kv);
    }
  }
  __syncthreads();

  // ---- merge the parked states.  The first wave with tiles leads the
  // segment the share starts inside; every wave leads the segment it ends
  // inside if that segment starts within the wave's part.  The contributors
  // of a segment are the waves whose parts meet it (with fewer tiles than
  // waves, each non-empty part is one tile); wave w keeps its piece in slot 0
  // if the segment began before its part, else in slot 1.  Leaders post
  // their tasks to LDS; then every thread of the workgroup merges.
  const int32_t first_wave = share_of(0, span, kNW);  // the wave whose part holds tile F0
  for (int k = 0; k < 2; ++k) {
    int32_t* task = tasks + (v * 2 + k) * kTaskInts;
    bool lead = false;
    Seg s{};
    if (G0 < G1) {
      s = seg_containing(PB, Ls, B, H_kv, k == 0 ? G0 : G1 - 1);
      lead = k == 0 ? (v == first_wave && s.S0 < F0) : (s.S1 > G1 && s.S0 >= G0);
    }
    if (lane == 0) task[0] = lead ? 1 : 0;
    if (!lead) continue;
    const int32_t lo = max(s.S0, F0), hi = min(s.S1, F1);
    const int32_t va = share_of(lo - F0, span, kNW);
    const int32_t nc = span >= kNW ? share_of(hi - 1 - F0, span, kNW) - va + 1 : hi - lo;
    if (lane < nc) {
      const int32_t w = span >= kNW ? va + lane : share_of(lo + lane - F0, span, kNW);
      task[kTaskHead + lane] = (w * 2 + (s.S0 < part_start(w) ? 0 : 1)) * slot_floats;
    }
    if (lane == 0) {
      task[1] = nc;
      task[2] = (s.b * H_kv + s.kvh) * G;                       // output row of head 0
      task[3] = (s.S0 >= F0 && s.S1 <= F1) ? -1 : 2 * wg + (s.S0 < F0 ? 0 : 1);  // partial slot
    }
  }
  pa::lds_barrier();
  for (int t = 0; t < 2 * kNW; ++t) {
    const int32_t* task = tasks + t * kTaskInts;
    if (task[0] == 0) continue;  // uniform
    const int32_t nc = task[1], orow = task[2], wslot = task[3];
    for (int32_t e = tid; e < G * D; e += kWG) {
      const int32_t g = e / D;
      const Merged x = merge_partials<kNW>(nc, [&](int32_t i, float& m, float& o, float& l) {
        const float* st = lds_st + task[kTaskHead + i];
        m = st[G * D + g];
        o = st[e];
        l = st[G * D + G + g];
      });
      if (wslot < 0) {
        store_out<BF16>(a.out, (int64_t)orow * D + e, x.acc / x.den);
      } else {
        // Partial for the merge kernel: (max, sum, unnormalised output).
        a.ws_o[(int64_t)wslot * G * D + e] = x.acc;
        if (e - g * D == 0) {
          a.ws_m[wslot * G + g] = x.mx;
          a.ws_l[wslot * G + g] = x.den;
        }
      }
    }
  }

  // ---- record for the partial-merge kernel: the segment this share ends
  // inside, if it also starts inside the share (this workgroup holds its
  // first part).
  if (tid == 0) {
    const Seg s = seg_containing(PB, Ls, B, H_kv, F1 - 1);
    const bool first = s.S1 > F1 && s.S0 >= F0;
    rec[0] = first ? 1 : 0;
    rec[1] = s.b;
    rec[2] = s.kvh;
    rec[3] = s.S0;
    rec[4] = s.S1;
    rec[5] = Tt;
  }
}

// Merges the partials of the segment recorded by workgroup blockIdx.x of
// the decode kernel (grid of W workgroups).  The contributors are the
// shares that meet the segment: consecutive shares from the recording one
// when every share is non-empty (T >= W), else one share per tile.  The
// first contributor's partial is in slot 2w + 1, every later one in slot 2w.
template <bool BF16, int D>
__global__ void __launch_bounds__(kMergeWG)
merge_kernel(DecodeArgs a) {
  __shared__ int32_t slots[kMaxWGs];
  const int32_t* rec = a.records + blockIdx.x * kRecInts;
  if (rec[0] == 0) return;
  const int32_t W = gridDim.x, G = a.G;
  const int32_t b = rec[1], kvh = rec[2], S0 = rec[3], S1 = rec[4], Tt = rec[5];
  const int32_t wa = blockIdx.x;
  // With one tile per non-empty share (T < W <= kMaxWGs), the share of tile
  // f is ((f + 1) W - 1) / T, small enough for 32-bit arithmetic.
  const int32_t n = Tt >= W ? share_of(S1 - 1, Tt, W) - wa + 1 : S1 - S0;
  for (int32_t i = threadIdx.x; i < n; i += kMergeWG) {
    const int32_t w = Tt >= W ? wa + i : ((S0 + i + 1) * W - 1) / Tt;
    slots[i] = 2 * w + (i == 0 ? 1 : 0);
  }
  __syncthreads();
  for (int32_t e = threadIdx.x; e < G * D; e += kMergeWG) {
    const int32_t g = e / D;
    const Merged x = merge_partials<8>(n, [&](int32_t i, float& m, float& o, float& l) {
      const int32_t slot = slots[i];
      m = a.ws_m[slot * G + g];
      o = a.ws_o[(int64_t)slot * G * D + e];
      l = a.ws_l[slot * G + g];
    });
    store_out<BF16>(a.out, ((int64_t)b * a.H_kv + kvh) * G * D + e, x.acc / x.den);
  }
}

// ----------------------------------------------------------- host helpers
int decode_wgs() {
  // Tuning override (read on every call): PA_DECODE_WGS = workgroups of
  // the decode grid.  Any value gives the same result up to fp32 rounding.
  const char* e = std::getenv("PA_DECODE_WGS");
  const int x = e ? std::atoi(e) : kDefaultWGs;
  return x >= 1 && x <= kMaxWGs ? x : kDefaultWGs;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct WorkspaceLayout {
  size_t rec_off, o_off, m_off, l_off, total;
};

WorkspaceLayout workspace_layout(const pa_cache_desc* d, int32_t H_q) {
  const size_t G = H_q / d->num_kv_heads;
  WorkspaceLayout w;
  w.rec_off = 0;
  w.o_off = align_up((size_t)kMaxWGs * kRecInts * sizeof(int32_t), 256);
  w.m_off = w.o_off + align_up((size_t)2 * kMaxWGs * G * d->head_dim * sizeof(float), 256);
  w.l_off = w.m_off + align_up((size_t)2 * kMaxWGs * G * sizeof(float), 256);
  w.total = w.l_off + align_up((size_t)2 * kMaxWGs * G * sizeof(float), 256);
  return w;
}

// Waves per workgroup and tiles in flight per wave, chosen so that the
// live registers stay under the budget of two waves per SIMD (one for the
// largest query groups).
template <bool BF16, int GP>
struct Config {
  static constexpr int kNW = GP >= 16 ? 4 : 8;
  static constexpr int NBUF = GP >= 8 ? 2 : (BF16 ? PA_DECODE_NB_BF16 : 2);
};

size_t lds_bytes(int nw, int32_t G, int32_t D, int32_t B) {
  return (size_t)nw * 2 * (G * D + 2 * G) * sizeof(float) +
         (size_t)(2 * B + 1 + nw + 2 * nw * (kTaskHead + nw)) * sizeof(int32_t);
}

template <bool BF16, int D, int GP>
pa_status launch(const DecodeArgs& a, hipStream_t s) {
  using C = Config<BF16, GP>;
  auto kern = a.log2_bs >= 4 ? decode_kernel<BF16, D, GP, C::kNW, C::NBUF, false>
                             : decode_kernel<BF16, D, GP, C::kNW, C::NBUF, true>;
  const size_t lds = lds_bytes(C::kNW, a.G, D, a.B);
  if (lds > kMaxLds)
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_decode: %d sequences need %zu bytes of LDS (> %zu)",
                    a.B, lds, kMaxLds);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess)
      return pa::fail(PA_ERR_DEVICE, "pa_decode: LDS attribute: %s", hipGetErrorString(e));
  }
  const int wgs = decode_wgs();
  hipLaunchKernelGGL(kern, dim3(wgs), dim3(C::kNW * kWave), lds, s, a);
  if (wgs > 1)
    hipLaunchKernelGGL((merge_kernel<BF16, D>), dim3(wgs), dim3(kMergeWG), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pa::fail(PA_ERR_DEVICE, "pa_decode: %s", hipGetErrorString(e));
  return PA_OK;
}

template <bool BF16, int D>
pa_status dispatch_g(const DecodeArgs& a, hipStream_t s) {
  if (a.G <= 1) return launch<BF16, D, 1>(a, s);
  if (a.G <= 2) return launch<BF16, D, 2>(a, s);
  if (a.G <= 4) return launch<BF16, D, 4>(a, s);
  if (a.G <= 8) return launch<BF16, D, 8>(a, s);
  return launch<BF16, D, 16>(a, s);
}

}  // namespace

extern "C" {

pa_status pa_supported(const pa_cache_desc* desc, int32_t num_q_heads) {
  pa_status st = pa::check_desc(desc);
  if (st != PA_OK) return st;
  if (num_q_heads < 1 || num_q_heads % desc->num_kv_heads)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "num_q_heads %d is not a multiple of %d",
                    num_q_heads, desc->num_kv_heads);
  const int32_t G = num_q_heads / desc->num_kv_heads;
  if (G > 16) return pa::fail(PA_ERR_UNSUPPORTED, "group size %d > 16", G);
  return PA_OK;
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
  if (num_seqs > kMaxSeqs)
    return pa::fail(PA_ERR_UNSUPPORTED, "num_seqs %d > %d", num_seqs, kMaxSeqs);
  *bytes = workspace_layout(desc, num_q_heads).total;
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
  if (num_seqs > kMaxSeqs)
    return pa::fail(PA_ERR_UNSUPPORTED, "num_seqs %d > %d", num_seqs, kMaxSeqs);
  const int64_t len_cap = (int64_t)max_blocks_per_seq * block_size;
  if (len_cap > INT32_MAX)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "max_blocks_per_seq * block_size overflows int32");
  // Flat tile indices (sequence, KV head, tile) must fit in int32.
  if ((int64_t)num_seqs * ((len_cap + kTile - 1) / kTile) * desc->num_kv_heads >= (1ll << 31))
    return pa::fail(PA_ERR_UNSUPPORTED, "num_seqs * tiles per sequence * KV heads >= 2^31");
  if (!std::isfinite(scale)) return pa::fail(PA_ERR_INVALID_ARGUMENT, "scale is not finite");
  if (num_seqs == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out || !workspace)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
  const WorkspaceLayout wl = workspace_layout(desc, num_q_heads);
  if (workspace_bytes < wl.total)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "workspace %zu bytes < %zu needed", workspace_bytes,
                    wl.total);
  char* ws = reinterpret_cast<char*>(workspace);
  DecodeArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.tables = block_tables;
  a.lens = context_lens;
  a.out = out;
  a.records = reinterpret_cast<int32_t*>(ws + wl.rec_off);
  a.ws_o = reinterpret_cast<float*>(ws + wl.o_off);
  a.ws_m = reinterpret_cast<float*>(ws + wl.m_off);
  a.ws_l = reinterpret_cast<float*>(ws + wl.l_off);
  a.B = num_seqs;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = desc->num_blocks;
  a.H_kv = desc->num_kv_heads;
  a.G = num_q_heads / desc->num_kv_heads;
  a.log2_bs = pa::ilog2_exact(block_size);
  a.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  hipStream_t s = (hipStream_t)stream;
  const bool bf16 = desc->dtype == PA_BF16;
  if (bf16 && desc->head_dim == 128) return dispatch_g<true, 128>(a, s);
  if (bf16) return dispatch_g<true, 64>(a, s);
  if (desc->head_dim == 128) return dispatch_g<false, 128>(a, s);
  return dispatch_g<false, 64>(a, s);
}

}  // extern "C"
