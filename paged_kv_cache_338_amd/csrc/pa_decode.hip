// Single-query (decode) attention that reads K/V through per-sequence block
// tables (gfx950 / CDNA4, wave64), in one kernel launch.
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
//  * A segment is one (KV head, sequence b) pair; it has ceil(L_b / 16)
//    tiles of 16 tokens.  All tiles are numbered in one flat, head-major
//    order (KV head, b, tile).  The T tiles are cut into equal shares, one
//    per workgroup, and each workgroup's share into equal sub-shares, one
//    per wave, so every wave streams the same number of K/V bytes whatever
//    the length mix.
//  * The dispatcher deals workgroups to the 8 XCDs in turn, so workgroups
//    blockIdx and blockIdx + 8 run on the same XCD (which XCD takes
//    blockIdx 0 varies from launch to launch).  Shares are therefore dealt
//    by blockIdx % 8 first: the workgroups of one XCD take consecutive
//    shares, and with a multiple of 8 KV heads every XCD owns whole heads,
//    so every segment's pieces are computed on one XCD.  Correctness does
//    not depend on this placement (see below); only the merge's speed does.
//  * Blocks of >= 16 tokens: a wave walks its sub-share as batches of up to
//    NBUF tiles; a batch holds the rest of one segment and, if that segment
//    ends inside it, the start of the next, so crossing a segment boundary
//    costs no extra round trip.  The block ids of the sub-share are fetched
//    64 tiles at a time by one vector load (lane i: tile i) and read with
//    v_readlane a batch ahead; each batch issues its segments' query rows and
//    all its tile loads before the first use.  Smaller blocks: one pipelined
//    piece per segment, block ids gathered per lane.
//  * A segment wholly inside a wave's sub-share is written out by the wave.
//    A piece cut by a sub-share boundary leaves its online-softmax state
//    (max, sum, unnormalised output) in LDS; after a barrier the workgroup
//    combines the pieces of each segment, writes the segments that lie
//    inside its share and publishes one partial state for each segment cut
//    by its share boundary (at most two).
//  * Cut segments are merged inside the kernel by the last workgroup to
//    publish a piece (a per-segment arrival counter; no workgroup ever waits
//    for another).  Pieces are published with device-scope stores, and the
//    counter also sums the XCD numbers of the contributors (and their
//    squares), read from the hardware.  When all of them ran on the
//    merger's XCD, every piece went through its L2 and is read from there;
//    otherwise the merger reads at device scope.  The merger restores the
//    counter to zero, so a zero-filled workspace stays ready for the next
//    call (graph replays included).
//  * Per tile (bf16 / fp16 pools): the K rows of the 16 tokens are the A
//    operand of a v_mfma_f32_16x16x32 chain whose B operand is the KV head's
//    G query rows, so the logits of head g and token 4j+r land in lane
//    16j+g, register r.  The probabilities, rounded to the pool's 16-bit
//    format, are the A operand of a v_mfma_f32_16x16x16 chain against the V
//    rows (D/16 output column blocks) and against a ones operand (the
//    softmax sums), so the output and its normaliser accumulate in MFMA
//    registers.  fp32 pools use v_mfma_f32_16x16x4_f32 for the logits and
//    the VALU for P*V, with the probabilities broadcast by DPP.
//  * The running max is raised lazily: only when a logit exceeds it by more
//    than 8 (log2 units) are the sum and output rescaled, so most tiles skip
//    the rescale.  Any reference value gives the same softmax.
//  * Blocks of >= 16 tokens are read through a buffer resource spanning the
//    tile; the padding tiles of the pipeline get a zero-length resource, so
//    every loop iteration issues the same loads and each use waits only for
//    its own tile.
//  * Masked positions (past the context length, only in a segment's tail
//    tile) get weight 0 and their V rows are zeroed, so garbage or NaN in
//    unused slots of a block cannot reach the output.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "pa_attn_tile.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace {

using pa::f32x2_t;
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
using pa::floatx4_t;
using pa::Geometry;
using pa::issue_tile;
using pa::issue_tile_small;
using pa::kTile;
using pa::kWave;
using pa::MfmaState;
using pa::TileRegs;
using pa::u32x4_t;
using pa::uni;
constexpr int kMaxWGs = 1024;     // grid bound: the workspace holds 2 pieces per workgroup
constexpr int kDefaultWGs = 256;  // one workgroup per compute unit
constexpr int kXcds = 8;          // XCDs of the part; workgroups are dealt to them in turn
constexpr int kMaxSeqs = 8192;    // lengths snapshot in LDS
constexpr int kMaxKvHeads = 4096; // a segment's (sequence, KV head) packs into 32 bits
constexpr int kNW = 4;            // waves per workgroup
constexpr int kWG = kNW * kWave;
constexpr int kSlots = 2 * kNW;   // LDS piece slots: two per wave
constexpr size_t kMaxLds = 160 * 1024;
// Cache-policy operand of the buffer intrinsics: device scope (sc1).
constexpr int kDeviceScope = 16;
#ifndef PA_DECODE_NB_BF16
#define PA_DECODE_NB_BF16 3  // tiles per batch for 16-bit pools (build-time tuning knob)
#endif
#ifndef PA_DECODE_MERGE_BATCH
#define PA_DECODE_MERGE_BATCH 8  // contributors' loads in flight per lane in the merge
#endif
#ifndef PA_DECODE_NB_APPEND
#define PA_DECODE_NB_APPEND 2  // the same when appending (its new-row reloads need registers)
#endif

struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* tables;
  const int32_t* lens;
  void* out;
  float* ws_o;        // [2 * kMaxWGs][G][D] published pieces: unnormalised output
  float* ws_ml;       // [2 * kMaxWGs][G][2] their reference max (log2 units) and sum
                      // of exp2(x - max), side by side so one 8-byte load fetches both
  uint64_t* counters;  // [H_kv * B] arrival counters, zero between calls
  const void* new_k;   // pa_decode_append: [B][H_kv][D] rows of each sequence's newest
  const void* new_v;   // token (position L - 1), written to the pools; else NULL
  int32_t B;
  int32_t max_blocks;
  int32_t num_blocks;
  int32_t H_kv;
  int32_t G;
  int32_t log2_bs;
  float scale_log2;  // scale * log2(e)

  __device__ pa::KvPool pool() const { return {k_cache, v_cache, num_blocks, H_kv, log2_bs}; }
};

template <bool k16, int D, int GP>
struct WaveState {
  using Geo = Geometry<k16, D>;
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

// One segment (KV head kvh, sequence b) and its flat tile range [S0, S1).
struct Seg {
  int32_t b, kvh, nt, L, S0, S1;
};

// Largest b in [0, B) with PB[b] <= r (PB: exclusive prefix sums of tiles
// per sequence, in LDS).  For r < PB[B] that is the non-empty sequence
// holding tile r of a head.
__device__ __forceinline__ int32_t find_seq(const int32_t* PB, int32_t B, int32_t r) {
  int32_t lo = 0, hi = B - 1;
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if (PB[mid] <= r) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// The segment holding flat tile f (0 <= f < H_kv * NT, NT = tiles per head);
// f is wave-uniform.
__device__ __forceinline__ Seg seg_containing(const int32_t* PB, const int32_t* Ls, int32_t B,
                                              int32_t H_kv, int32_t NT, int32_t f) {
  Seg s;
  s.kvh = uni(min(static_cast<int32_t>(static_cast<uint32_t>(f) / static_cast<uint32_t>(NT)),
                  H_kv - 1));
  const int32_t r = f - s.kvh * NT;
  s.b = uni(find_seq(PB, B, r));
  const int32_t pb = uni(PB[s.b]);
  s.nt = max(uni(PB[s.b + 1]) - pb, 1);
  s.S0 = s.kvh * NT + pb;
  s.S1 = s.S0 + s.nt;
  s.L = uni(Ls[s.b]);
  return s;
}

// Moves s to the next non-empty segment in flat order.  Called only while
// one exists; should the snapshot say otherwise, s becomes an empty segment
// at the end of every range, which stops every loop that walks segments.
__device__ __forceinline__ void seg_advance(Seg& s, const int32_t* PB, const int32_t* Ls,
                                            int32_t B, int32_t H_kv, int32_t NT) {
  // The next sequence with tiles, in this head or a later one (the empty
  // sequences of a head are the same in every head).
  int32_t b = s.b + 1;
  while (b < B && uni(PB[b + 1]) == uni(PB[b])) ++b;
  int32_t kvh = s.kvh;
  if (b >= B) {
    b = 0;
    while (b < B && uni(PB[b + 1]) == uni(PB[b])) ++b;
    ++kvh;
  }
  const bool end = kvh >= H_kv || b >= B;
  b = min(b, B - 1);
  const int32_t pb = uni(PB[b]);
  s.b = b;
  s.kvh = kvh;
  s.nt = uni(PB[b + 1]) - pb;
  s.S0 = end ? 0x7FFFFFFF : kvh * NT + pb;
  s.S1 = end ? 0x7FFFFFFF : s.S0 + s.nt;
  s.L = uni(Ls[b]);
}

template <int E, int D, int GP>
__device__ __forceinline__ void consume_tile(WaveState<(E != 0), D, GP>& st,
                                             const TileRegs<(E != 0), D>& r, const u32x4_t* qf,
                                             const float* qf32, float scale_log2, int32_t t0,
                                             int32_t end, int lane) {
  using Geo = Geometry<(E != 0), D>;
  floatx4_t s = {0.f, 0.f, 0.f, 0.f};
  if constexpr (E != 0) {
#pragma unroll
    for (int p = 0; p < Geo::kKPieces; ++p) s = pa::mfma_k32<E>(r.k[p], qf[p], s);
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
      if constexpr (E != 0) {
        vf[q][2 * w] = ok ? pa::lo16<E>(r.v[q][w]) : 0.f;
        vf[q][2 * w + 1] = ok ? pa::hi16<E>(r.v[q][w]) : 0.f;
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

// kSplit: take the unmasked variant for whole tiles (a uniform branch);
// otherwise always mask (one code copy, for register-tight callers).
template <int E, int D, bool kSplit>
__device__ __forceinline__ void consume_tile_mfma(MfmaState<D>& st, const TileRegs<true, D>& r,
                                                  const u32x4_t* qf, float scale_log2,
                                                  int32_t t0, int32_t end, int lane) {
  if (kSplit && t0 + kTile <= end)
    pa::consume_tile_mfma_impl<E, D, false>(st, r, qf, scale_log2, t0, end - 1, end, lane);
  else
    pa::consume_tile_mfma_impl<E, D, true>(st, r, qf, scale_log2, t0, end - 1, end, lane);
}

// Loads the G query rows of segment (b, kvh) as the MFMA B operand (lane
// 16j + g holds 16-byte pieces of head g; zero for g >= G).
template <bool k16, int D>
__device__ __forceinline__ void load_q(const DecodeArgs& a, int32_t b, int32_t kvh, u32x4_t* qf,
                                       float* qf32, int lane) {
  using Geo = Geometry<k16, D>;
  const int jr = lane >> 4, c16 = lane & 15;
  const bool live = c16 < a.G;
  const int64_t row = ((int64_t)b * a.H_kv + kvh) * a.G + (live ? c16 : 0);
  const char* qb = reinterpret_cast<const char*>(a.q) + row * Geo::kRowBytes + jr * 16;
#pragma unroll
  for (int p = 0; p < Geo::kKPieces; ++p) {
    u32x4_t x = *reinterpret_cast<const u32x4_t*>(qb + p * 64);
    if (!live) x = u32x4_t{0, 0, 0, 0};
    if constexpr (k16) {
      qf[p] = x;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) qf32[4 * p + e] = pa::as_float(x[e]);
    }
  }
}

// Largest w with floor(T * w / W) <= f: the share (of W equal shares of T
// units) that holds unit f, for 0 <= f < T < 2^31 and W <= 2^10, i.e.
// floor(((f + 1) W - 1) / T).  The quotient comes from one double division
// (its operands, below 2^41, are exact) and one integer check fixes the
// rounding; a 64-bit integer division would be a long software sequence on
// the critical path of the merge.
__device__ __forceinline__ int32_t share_of(int32_t f, int32_t T, int32_t W) {
  const int64_t x = ((int64_t)f + 1) * W - 1;
  int32_t w = static_cast<int32_t>(static_cast<double>(x) / static_cast<double>(T));
  if ((int64_t)w * T > x) --w;
  else if ((int64_t)(w + 1) * T <= x) ++w;
  return w;
}

template <int E>
__device__ __forceinline__ void store_out(void* out, int64_t i, float x) {
  if constexpr (E != 0) reinterpret_cast<uint16_t*>(out)[i] = pa::round16<E>(x);
  else reinterpret_cast<float*>(out)[i] = x;
}

// Four output values of one head row, rounded once, stored with one write.
template <int E>
__device__ __forceinline__ void store_out4(void* out, int64_t i, floatx4_t x) {
  if constexpr (E != 0) {
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + i) =
        uint2{pa::pack2<E>(x[0], x[1]), pa::pack2<E>(x[2], x[3])};
  } else {
    *reinterpret_cast<floatx4_t*>(reinterpret_cast<float*>(out) + i) = x;
  }
}

// XCD the running workgroup was placed on (hardware register XCC_ID, bits
// 3:0).
__device__ __forceinline__ int32_t xcd_id() {
  return static_cast<int32_t>(__builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 0xF);
}

// LDS of the workgroup step: one piece slot per (wave, end of its
// sub-share) with its unnormalised output, reference max and sum, and the
// slot's segment.
template <int D, int GP>
struct LdsPieces {
  float o[kSlots][GP][D];
  float m[kSlots][GP];
  float l[kSlots][GP];
  int4 seg[kSlots];        // S0, S1, b | kvh << 16 (kvh < 2^15), valid: one 16-byte read
  int32_t flag[2];         // per published piece: 0 not last, 1 merge from L2, 2 at device scope
  int32_t la[2], n[2];     // per published piece: its segment's first contributor and count
};

template <int E, int D, int GP, int NBUF, bool kSmall, bool kAppend, bool kNT>
__global__ void __launch_bounds__(kWG)
__attribute__((amdgpu_waves_per_eu(kSmall ? (((E != 0) || GP * D < 16 * 128) ? 2 : 1)
                                          : ((E != 0) ? 2 : 1))))
decode_kernel(DecodeArgs a) {
  constexpr bool BF16 = E != 0;  // 16-bit pools (bf16 or fp16)
  using Geo = Geometry<BF16, D>;
  using Pieces = LdsPieces<D, GP>;
  constexpr int kC4 = D / 4;  // 4-column groups of a head row
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), v = tid >> 6;
  const int jr = lane >> 4, c16 = lane & 15;
  const int32_t bx = blockIdx.x, nwg = gridDim.x;
  const int32_t B = a.B, H_kv = a.H_kv, G = a.G, H_q = H_kv * G;

  // LDS: the pieces, then the lengths snapshot and its prefix sums.
  Pieces& P = *reinterpret_cast<Pieces*>(smem);
  int32_t* PB = reinterpret_cast<int32_t*>(smem + sizeof(Pieces));  // [B + 1]
  int32_t* Ls = PB + B + 1;                                          // [B]
  int32_t* misc = Ls + B;                                            // [kNW]

  if (lane < 2) P.seg[2 * v + lane] = int4{0, 0, 0, 0};

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
    if (b < B) PB[b] = pre + incl - nt;
    carry += tot;
    __syncthreads();
  }
  if (tid == 0) PB[B] = carry;
  __syncthreads();

  const int32_t NT = uni(PB[B]);  // tiles per KV head
  const int32_t Tt = NT * H_kv;   // flat tiles (host bounds it below 2^31)

  // Sequences with no context get a zero row (workgroup b % W writes it).
  for (int32_t b = bx; b < B; b += nwg) {
    if (Ls[b] == 0) {
      for (int32_t e = tid; e < H_q * D; e += kWG)
        store_out<E>(a.out, (int64_t)b * H_q * D + e, 0.f);
    }
  }
  if (Tt == 0) return;

  if constexpr (kAppend) {
    // ---- the newest tokens' rows into the pools, spread over the waves of
    // the grid at its start: pair p = (sequence b, KV head) goes to wave p
    // mod W, 16 bytes per lane (K rows in the first half of a pair's lanes,
    // V rows in the second).  The waves that read these rows take them from
    // new_k / new_v, so nothing in this launch waits for the writes.
    constexpr int kChunks = Geo::kRowBytes / 16;               // per row
    constexpr int kPairsPerPass = kWave / (2 * kChunks) > 0 ? kWave / (2 * kChunks) : 1;
    constexpr int kLanesPerPair = 2 * kChunks > kWave ? kWave : 2 * kChunks;
    const int32_t npairs = B * H_kv, W = nwg * kNW;
    const int32_t gw = bx * kNW + v;
    const int pl = lane % kLanesPerPair;      // lane within its pair
    const int pk = lane / kLanesPerPair;      // pair within the pass
    for (int32_t p0 = gw * kPairsPerPass; p0 < npairs; p0 += W * kPairsPerPass) {
      const int32_t p = p0 + pk;
      if (p < npairs && pk < kPairsPerPass) {
        const int32_t b = p / H_kv, kvh = p - b * H_kv;
        const int32_t L = Ls[b];
        if (L > 0) {
          const int32_t e = min((L - 1) >> a.log2_bs, a.max_blocks - 1);
          const int32_t phys = a.tables[(int64_t)b * a.max_blocks + e];
          if (phys >= 0 && phys < a.num_blocks) {
            const int64_t dst = ((((int64_t)phys * H_kv + kvh) << a.log2_bs) +
                                 ((L - 1) & ((1 << a.log2_bs) - 1))) * Geo::kRowBytes;
            const int64_t src = (int64_t)p * Geo::kRowBytes;
            // One row per half of the pair's lanes; rows of more than 64
            // chunks (none here) would need more lanes.
            for (int c = pl; c < 2 * kChunks; c += kLanesPerPair) {
              const bool isv = c >= kChunks;
              const int off = (isv ? c - kChunks : c) * 16;
              const char* sp = reinterpret_cast<const char*>(isv ? a.new_v : a.new_k) + src + off;
              char* dp = reinterpret_cast<char*>(const_cast<void*>(isv ? a.v_cache : a.k_cache)) +
                         dst + off;
              *reinterpret_cast<u32x4_t*>(dp) = *reinterpret_cast<const u32x4_t*>(sp);
            }
          }
        }
      }
    }
  }

  // ---- shares.  Logical workgroup lw takes share [T*lw/W, T*(lw+1)/W);
  // with W a multiple of 8 the workgroups with blockIdx = x mod 8 (one XCD)
  // take the consecutive logical indices x*W/8 .. (x+1)*W/8 - 1.
  const int32_t per_xcd = nwg % kXcds == 0 ? nwg / kXcds : 0;
  const int32_t lw = per_xcd ? (bx % kXcds) * per_xcd + bx / kXcds : bx;
  // floor(Tt * w / nwg) in 32-bit arithmetic: Tt = qt * nwg + rt with
  // rt < nwg <= 1024, so rt * w < 2^21.
  const uint32_t qt = static_cast<uint32_t>(Tt) / static_cast<uint32_t>(nwg);
  const uint32_t rt = static_cast<uint32_t>(Tt) - qt * static_cast<uint32_t>(nwg);
  auto bound = [&](uint32_t w) {
    return static_cast<int32_t>(qt * w + rt * w / static_cast<uint32_t>(nwg));
  };
  const int32_t A0 = uni(bound(lw)), A1 = uni(bound(lw + 1));
  const int32_t G0 = uni(A0 + static_cast<int32_t>((int64_t)(A1 - A0) * v / kNW));
  const int32_t G1 = uni(A0 + static_cast<int32_t>((int64_t)(A1 - A0) * (v + 1) / kNW));
  const int log2_bs = a.log2_bs;
  const int nbt = log2_bs >= 4 ? 1 : (kTile >> log2_bs);  // table lanes per tile
  const int tpc_log = log2_bs >= 4 ? 6 : 2 + log2_bs;       // log2(tiles per table chunk)

  using State = std::conditional_t<BF16, MfmaState<D>, WaveState<false, D, GP>>;
  // Finishes segment s after its last tile in this wave's sub-share.  A
  // segment wholly inside the sub-share is written out; a cut piece leaves
  // (max, sum, unnormalised output) in LDS slot 2v + 0 if the segment began
  // before the sub-share, else 2v + 1.
  auto finish = [&](const State& st, const Seg s) {
    const bool whole = s.S0 >= G0 && s.S1 <= G1;
    const int slot = 2 * v + (s.S0 < G0 ? 0 : 1);
    if (!whole && lane == 0) P.seg[slot] = int4{s.S0, s.S1, s.b | (s.kvh << 16), 1};
    if constexpr (BF16) {
      // The accumulators already hold whole tiles (lane 16j + c, register
      // r: head 4j + r, columns kBlk*c .. kBlk*c + kBlk - 1).
      constexpr int kBlk = D / 16;
      pa::static_for<0, 4>([&](auto Q) {
        constexpr int q = decltype(Q)::value;
        const int g = 4 * jr + q;
        const float lg = st.l[q];  // head g's sum
        if (g < G) {
          if (whole) {
            const float inv = 1.f / lg;
            uint32_t pk[kBlk / 2];
#pragma unroll
            for (int i = 0; i < kBlk / 2; ++i)
              pk[i] = pa::pack2<E>(st.acc[2 * i][q] * inv, st.acc[2 * i + 1][q] * inv);
            char* dst = reinterpret_cast<char*>(a.out) +
                        ((((int64_t)s.b * H_kv + s.kvh) * G + g) * D + kBlk * c16) * 2;
            if constexpr (kBlk == 8) *reinterpret_cast<u32x4_t*>(dst) = u32x4_t{pk[0], pk[1], pk[2], pk[3]};
            else *reinterpret_cast<uint2*>(dst) = uint2{pk[0], pk[1]};
          } else {
            float* dst = &P.o[slot][g][kBlk * c16];
#pragma unroll
            for (int i = 0; i < kBlk; i += 4)
              *reinterpret_cast<floatx4_t*>(dst + i) =
                  floatx4_t{st.acc[i][q], st.acc[i + 1][q], st.acc[i + 2][q], st.acc[i + 3][q]};
            if (c16 == 0) P.l[slot][g] = lg;
          }
        }
      });
      if (!whole && lane < G) P.m[slot][lane] = st.ref;
    } else {
      // ---- merge the 4 row states (lanes g, 16+g, 32+g, 48+g hold head g)
      const float M = pa::rows_max(st.m);
      const float sc = exp2f(st.m - M);
      const float lt = pa::rows_sum(st.l * sc);
      pa::static_for<0, GP>([&](auto gi) {
        constexpr int g = decltype(gi)::value;
        const float f = pa::row_bcast<g>(sc);
        const float inv = 1.f / pa::row_bcast<g>(lt);
        float o[Geo::kCols];
#pragma unroll
        for (int c = 0; c < Geo::kCols; ++c) o[c] = pa::rows_sum(st.o[g][c] * f);
        if (g < G && (g & 3) == jr) {
          if (whole) {
            const int64_t base = (((int64_t)s.b * H_kv + s.kvh) * G + g) * D + c16 * Geo::kCols;
#pragma unroll
            for (int c = 0; c < Geo::kCols; ++c) store_out<E>(a.out, base + c, o[c] * inv);
          } else {
#pragma unroll
            for (int c = 0; c < Geo::kCols; ++c) P.o[slot][g][c16 * Geo::kCols + c] = o[c];
          }
        }
      });
      if (!whole && lane < G) {
        P.m[slot][lane] = M;
        P.l[slot][lane] = lt;
      }
    }
  };

  if (G0 < G1) {
    State st;
    st.reset();
    if constexpr (!kSmall) {
      // ---- the sub-share as a stream of batches of up to NBUF tiles.  A
      // batch holds the remaining tiles of one segment A and, if A ends
      // inside it, the first tiles of the next segment B, so a sub-share that
      // crosses a segment boundary costs no extra round trip.  The query rows
      // of A and B are loaded with the batch's tiles.
      struct Batch {
        Seg A, B;
        int32_t fa;      // flat index of the batch's first tile (in A)
        int32_t nA, n;   // tiles of A; tiles in all (the rest are B's)
        bool endA, endB; // the segment's last tile in this sub-share is here
      };
      Seg cs = seg_containing(PB, Ls, B, H_kv, NT, G0);
      int32_t f = G0;  // next flat tile of the sub-share
      auto next = [&]() {
        Batch bt;
        bt.A = cs;
        bt.B = cs;
        bt.fa = f;
        // An exhausted cursor (S0 past f) yields an empty batch.
        const int32_t limA = min(cs.S1, G1);
        bt.nA = cs.S0 <= f ? max(min(NBUF, limA - f), 0) : 0;
        bt.endA = bt.nA > 0 && f + bt.nA == limA;
        f += bt.nA;
        bt.n = bt.nA;
        if (bt.nA > 0 && f == cs.S1 && f < G1) {
          seg_advance(cs, PB, Ls, B, H_kv, NT);
          if (bt.nA < NBUF && cs.S0 == f) {
            bt.B = cs;
            const int32_t limB = min(cs.S1, G1);
            const int32_t nB = min(NBUF - bt.nA, limB - f);
            bt.endB = f + nB == limB;
            f += nB;
            bt.n += nB;
            if (f == cs.S1 && f < G1) seg_advance(cs, PB, Ls, B, H_kv, NT);
          }
        }
        if (bt.n == bt.nA) bt.endB = false;
        return bt;
      };
      // Segment and in-segment tile of batch slot u.
      auto slot_tile = [&](const Batch& bt, int u, int32_t& kvh, int32_t& t) {
        const int32_t uu = min(u, max(bt.n - 1, 0));
        const bool inA = uu < bt.nA;
        kvh = inA ? bt.A.kvh : bt.B.kvh;
        t = bt.fa + uu - (inA ? bt.A.S0 : bt.B.S0);
      };
      // Block ids of the sub-share, 64 tiles at a time: lane i of chunk c
      // holds the physical block of flat tile G0 + 64c + i (clamped to the
      // sub-share), found by a per-lane search of the lengths snapshot and one
      // vector load from the table, so batches read their block ids from
      // registers and the table is never on a batch's critical path.
      // Indices are clamped into the table so that no snapshot, however
      // inconsistent, can send a read outside it.
      auto chunk_phys = [&](int32_t c) -> int32_t {
        const int32_t fl = min(G0 + 64 * c + lane, G1 - 1);
        const int32_t kvh = min(static_cast<int32_t>(static_cast<uint32_t>(fl) /
                                                     static_cast<uint32_t>(NT)),
                                H_kv - 1);
        const int32_t r = fl - kvh * NT;
        const int32_t b = find_seq(PB, B, r);
        const int32_t t = r - PB[b];
        const int32_t e = min(max((t * kTile) >> log2_bs, 0), a.max_blocks - 1);
        return a.tables[(int64_t)b * a.max_blocks + e];
      };
      int32_t cbase = G0;  // flat tile of lane 0 of chunk `cur`
      int32_t cur = chunk_phys(0), nxt = 0;
      if (G1 - G0 > 64) nxt = chunk_phys(1);  // read only by sub-shares of more than 64 tiles
      // Block ids of a batch's tiles, read from the chunks into SGPRs.
      // They are taken for batch k+1 before batch k is consumed, when the
      // chunks are known to have arrived, so that the loop head waits for
      // nothing before issuing the next batch.
      auto batch_phys = [&](const Batch& bt, int32_t (&ph)[NBUF]) {
#pragma unroll
        for (int u = 0; u < NBUF; ++u) {
          const int32_t i = uni(min(bt.fa + min(u, max(bt.n - 1, 0)) - cbase, 127));
          ph[u] = i < 64 ? __builtin_amdgcn_readlane(cur, i) : __builtin_amdgcn_readlane(nxt, i - 64);
        }
      };
      Batch bt = next();
      int32_t ph[NBUF];
      batch_phys(bt, ph);
      while (true) {
        u32x4_t qa[Geo::kQRegs], qb[Geo::kQRegs];
        float qa32[Geo::kQF32], qb32[Geo::kQF32];
        load_q<BF16, D>(a, bt.A.b, bt.A.kvh, qa, qa32, lane);
        load_q<BF16, D>(a, bt.B.b, bt.B.kvh, qb, qb32, lane);
        TileRegs<BF16, D> buf[NBUF];
#pragma unroll
        for (int u = 0; u < NBUF; ++u) {
          int32_t kvh, t;
          slot_tile(bt, u, kvh, t);
          if constexpr (kAppend) {
            // The tile holding a segment's newest token (its last tile)
            // reads that row from the token's own rows.
            const bool inA = u < bt.nA;
            const int32_t S1 = inA ? bt.A.S1 : bt.B.S1, L = inA ? bt.A.L : bt.B.L;
            const int32_t b = inA ? bt.A.b : bt.B.b;
            issue_tile<BF16, D, kNT>(buf[u], a.pool(), ph[u], t, kvh, lane, u < bt.n);
            if (u < bt.n && bt.fa + u == S1 - 1) {  // uniform
              const int64_t src = ((int64_t)b * H_kv + kvh) * Geo::kRowBytes;
              pa::reload_new_row<BF16, D>(buf[u], (L - 1) & (kTile - 1),
                                          reinterpret_cast<const char*>(a.new_k) + src,
                                          reinterpret_cast<const char*>(a.new_v) + src, lane);
            }
            continue;
          }
          issue_tile<BF16, D, kNT>(buf[u], a.pool(), ph[u], t, kvh, lane, u < bt.n);
        }
        const Batch nx = next();
        batch_phys(nx, ph);
        if (nx.n > 0 && nx.fa + nx.n - 1 + NBUF - cbase >= 128) {
          // The batch after nx may leave the window [cbase, cbase + 128):
          // slide it by one chunk now, a batch ahead, so that a chunk is
          // never read in the iteration that loads it (batches are shorter
          // than a chunk, so that batch lies inside the new window).
          cbase += 64;
          cur = nxt;
          nxt = chunk_phys((cbase - G0) / 64 + 1);
        }
        // Keep every load of the batch ahead of the first use: left alone,
        // the scheduler sinks loads next to their uses to save registers.
        __builtin_amdgcn_sched_barrier(0);
        pa::static_for<0, NBUF>([&](auto U) {
          constexpr int u = decltype(U)::value;
          if (u < bt.nA) {
            const int32_t tok0 = kTile * (bt.fa + u - bt.A.S0);
            if constexpr (BF16) consume_tile_mfma<E, D, true>(st, buf[u], qa, a.scale_log2, tok0, bt.A.L, lane);
            else consume_tile<E, D, GP>(st, buf[u], qa, qa32, a.scale_log2, tok0, bt.A.L, lane);
          }
        });
        if (bt.endA) {
          finish(st, bt.A);
          st.reset();
        }
        pa::static_for<0, NBUF>([&](auto U) {
          constexpr int u = decltype(U)::value;
          if (u >= bt.nA && u < bt.n) {
            const int32_t tok0 = kTile * (bt.fa + u - bt.B.S0);
            if constexpr (BF16) consume_tile_mfma<E, D, true>(st, buf[u], qb, a.scale_log2, tok0, bt.B.L, lane);
            else consume_tile<E, D, GP>(st, buf[u], qb, qb32, a.scale_log2, tok0, bt.B.L, lane);
          }
        });
        if (bt.endB) {
          finish(st, bt.B);
          st.reset();
        }
        if (nx.n == 0) break;
        bt = nx;
      }
    } else {
      // ---- blocks smaller than a tile: the sub-share as pieces, one per
      // segment, each a pipelined loop over its tiles.
      Seg s = seg_containing(PB, Ls, B, H_kv, NT, G0);
      while (true) {
        const int32_t t0 = max(s.S0, G0) - s.S0;
        const int32_t n = min(s.S1, G1) - s.S0 - t0;
        u32x4_t qf[Geo::kQRegs];
        float qf32[Geo::kQF32];
        load_q<BF16, D>(a, s.b, s.kvh, qf, qf32, lane);
        TileRegs<BF16, D> buf[NBUF];
        auto consume = [&](const TileRegs<BF16, D>& r, int32_t j) {
          const int32_t tok0 = kTile * (t0 + j);
          const int32_t end = j < n ? s.L : tok0;  // padding: every row masked
          if constexpr (BF16) consume_tile_mfma<E, D, false>(st, r, qf, a.scale_log2, tok0, end, lane);
          else consume_tile<E, D, GP>(st, r, qf, qf32, a.scale_log2, tok0, end, lane);
        };
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
          if constexpr (kAppend) {
            if (j < n && t0 + jj == s.nt - 1) {  // uniform: the segment's last tile
              const int64_t src = ((int64_t)s.b * H_kv + s.kvh) * Geo::kRowBytes;
              issue_tile_small<BF16, D, kNT>(r, a.pool(), dA, jj - (c << tpc_log), t0 + jj, s.kvh,
                                             s.L, nbt, lane, (s.L - 1) & (kTile - 1),
                                        reinterpret_cast<const char*>(a.new_k) + src,
                                        reinterpret_cast<const char*>(a.new_v) + src);
              return;
            }
          }
          issue_tile_small<BF16, D, kNT>(r, a.pool(), dA, jj - (c << tpc_log), t0 + jj, s.kvh, s.L,
                                         nbt, lane);
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
        finish(st, s);
        if (s.S1 >= G1) break;
        st.reset();
        seg_advance(s, PB, Ls, B, H_kv, NT);
      }
    }
  }

  // ---- workgroup step: combine the pieces each segment left in LDS.
  __syncthreads();
  // Slots in flat order (slot 2v holds the piece at the start of wave v's
  // sub-share, 2v + 1 the one at its end); the valid slots of one segment
  // form a run.  The descriptors are read once into registers (every
  // thread reads the same values, so the control flow below is uniform)
  // and the slots are walked in one unrolled pass: a piece joins the
  // running state of its run by the rescaled-sum rule, and at the end of a
  // run the state is written out (segment inside the share) or published.
  // At most two runs reach past the share (the one holding its first tile
  // and the one holding its last); their states are published in piece slot
  // 2 lw (began before the share) or 2 lw + 1, at device scope.
  // The eight descriptors are read at once.  Bit k of vmask: slot k holds
  // a piece; of emask: it ends a run (the next valid slot holds another
  // segment).  Masks rather than arrays indexed at run time, which would live
  // in scratch memory.
  int4 dsc[kSlots];
#pragma unroll
  for (int k = 0; k < kSlots; ++k) dsc[k] = P.seg[k];
  uint32_t vmask = 0, emask = 0;
  {
    int32_t nextS0 = -1;  // S0 of the next valid slot (-1: none)
#pragma unroll
    for (int k = kSlots - 1; k >= 0; --k) {
      if (dsc[k].w) {
        vmask |= 1u << k;
        if (nextS0 != dsc[k].x) emask |= 1u << k;
        nextS0 = dsc[k].x;
      }
    }
  }
  // The published runs (S0, S1, b | kvh << 16) in scalars, assigned by
  // selects (a dynamically indexed array, or a reference to either set,
  // would live in scratch memory).
  int32_t pub_n = 0;
  int32_t p0S0 = 0, p0S1 = 0, p0bh = 0, p1S0 = 0, p1S1 = 0, p1bh = 0;
#pragma unroll
  for (int k = 0; k < kSlots; ++k) {
    if ((emask >> k & 1) && !(dsc[k].x >= A0 && dsc[k].y <= A1)) {  // uniform
      const bool first = pub_n == 0;
      p0S0 = first ? dsc[k].x : p0S0;
      p0S1 = first ? dsc[k].y : p0S1;
      p0bh = first ? dsc[k].z : p0bh;
      p1S0 = first ? p1S0 : dsc[k].x;
      p1S1 = first ? p1S1 : dsc[k].y;
      p1bh = first ? p1bh : dsc[k].z;
      ++pub_n;
    }
  }
  // Each thread combines one (head, 4-column group) item of every run: the
  // slots' values are read once, then each run takes the slots of its mask
  // (selects, not multiplications, keep the garbage of unused slots out).
  // The code is kept short: at the end of the kernel each SIMD runs one
  // wave, and every instruction on this path costs its full latency.
  for (int32_t e = tid; e < G * kC4; e += kWG) {
    const int32_t g = e / kC4, c4 = e - g * kC4;
    float sm[kSlots], sl[kSlots];
    floatx4_t so[kSlots];
#pragma unroll
    for (int k = 0; k < kSlots; ++k) {
      sm[k] = P.m[k][g];
      sl[k] = P.l[k][g];
      so[k] = *reinterpret_cast<const floatx4_t*>(&P.o[k][g][4 * c4]);
    }
    for (uint32_t rest = vmask; rest != 0;) {  // one run per iteration (uniform)
      const int k0 = __builtin_ctz(rest);
      const int k1 = __builtin_ctz(emask & ~((1u << k0) - 1));  // its last slot
      const uint32_t rm = vmask & ((2u << k1) - 1) & ~((1u << k0) - 1);
      rest &= ~((2u << k1) - 1);
      float M = -3.0e38f;
#pragma unroll
      for (int k = 0; k < kSlots; ++k) M = (rm >> k & 1) ? fmaxf(M, sm[k]) : M;
      floatx4_t O = {0.f, 0.f, 0.f, 0.f};
      float Lsum = 0.f;
#pragma unroll
      for (int k = 0; k < kSlots; ++k) {
        const bool in = rm >> k & 1;
        const float w = __builtin_amdgcn_exp2f(sm[k] - M);
        const floatx4_t x = w * so[k];
        O[0] += in ? x[0] : 0.f;
        O[1] += in ? x[1] : 0.f;
        O[2] += in ? x[2] : 0.f;
        O[3] += in ? x[3] : 0.f;
        Lsum += in ? w * sl[k] : 0.f;
      }
      const int4 d = P.seg[k1];
      const int32_t S0 = d.x, S1 = d.y, b = d.z & 0xFFFF, kvh = d.z >> 16;
      if (S0 >= A0 && S1 <= A1) {
        store_out4<E>(a.out, (((int64_t)b * H_kv + kvh) * G + g) * D + 4 * c4, O * (1.f / Lsum));
      } else {
        // Published written through to memory, so that the merger can read
        // it from any XCD.
        const int32_t ps = 2 * lw + (S0 < A0 ? 0 : 1);
        const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
            a.ws_o + (int64_t)ps * G * D, 0, G * D * 4, pa::kRsrcWord3);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, O), ro,
                                               (g * D + 4 * c4) * 4, 0, kDeviceScope);
        if (c4 == 0) {
          const __amdgpu_buffer_rsrc_t rml = __builtin_amdgcn_make_buffer_rsrc(
              a.ws_ml + (int64_t)ps * G * 2, 0, G * 8, pa::kRsrcWord3);
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, f32x2_t{M, Lsum}),
                                                rml, g * 8, 0, kDeviceScope);
        }
      }
    }
  }
  pub_n = min(pub_n, 2);
  if (pub_n == 0) return;  // uniform

  // ---- publish: the pieces are complete at device scope before the
  // arrival is counted.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  // Contributors of published run j: the logical workgroups la.. whose
  // shares meet the segment, n of them (one per tile when there are fewer
  // tiles than workgroups).
  if (tid < pub_n) {
    const int32_t S0 = tid == 0 ? p0S0 : p1S0, S1 = tid == 0 ? p0S1 : p1S1;
    const int32_t bh = tid == 0 ? p0bh : p1bh, b = bh & 0xFFFF, kvh = bh >> 16;
    const int32_t la = share_of(S0, Tt, nwg);
    const int32_t n = Tt >= nwg ? share_of(S1 - 1, Tt, nwg) - la + 1 : S1 - S0;
    P.la[tid] = la;  // for the merge, should this workgroup be last
    P.n[tid] = n;
    // Arrival: the count in bits 0-15, the sum of the contributors' XCD
    // numbers x in bits 16-31 and of x^2 in bits 32-47 (n <= 1024, x <= 7).
    // The n contributors ran on one XCD iff n * sum(x^2) = sum(x)^2, and on
    // this one iff moreover sum(x) = n * x.
    const uint64_t x = static_cast<uint64_t>(xcd_id());
    const uint64_t inc = 1 + (x << 16) + ((x * x) << 32);
    uint64_t* ctr = a.counters + (int64_t)kvh * B + b;
    const uint64_t tot = __hip_atomic_fetch_add(ctr, inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + inc;
    const uint64_t cnt = tot & 0xFFFF, s1 = (tot >> 16) & 0xFFFF, s2 = (tot >> 32) & 0xFFFF;
    const bool last = cnt == static_cast<uint64_t>(n);
    if (last) __hip_atomic_store(ctr, uint64_t{0}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool here = cnt * s2 == s1 * s1 && s1 == cnt * x;
    P.flag[tid] = last ? (here ? 1 : 2) : 0;
  }
  __syncthreads();

  // ---- the last contributor merges: out = sum_i 2^(m_i - M) o_i /
  // sum_i 2^(m_i - M) l_i over the pieces in flat order (so the result does
  // not depend on which workgroup arrived last), rounded once.  Pieces that
  // all went through this XCD's L2 are read from there; otherwise at device
  // scope.  Both published runs (if this workgroup is last for both) are
  // merged together, so their loads are in flight at once.  The kC4 lanes
  // that share a head each fetch one contributor's (max, sum) and pass them
  // round by shuffles, so a lane issues one 8-byte load per kC4
  // contributors besides its 16-byte output loads.
  const int32_t f0 = P.flag[0], f1 = pub_n > 1 ? P.flag[1] : 0;
  const int nm = (f0 ? 1 : 0) + (f1 ? 1 : 0);
  if (nm == 0) return;  // uniform
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(a.ws_o, 0, 0x7FFFFFFF, pa::kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rml = __builtin_amdgcn_make_buffer_rsrc(a.ws_ml, 0, 0x7FFFFFFF, pa::kRsrcWord3);
  const int32_t sub = lane & (kC4 - 1), base = lane - sub;  // lane within its head's group
  for (int32_t e0 = 0; e0 < nm * G * kC4; e0 += kWG) {  // uniform
    const int32_t e = min(e0 + tid, nm * G * kC4 - 1);  // spare lanes repeat the last item
    const bool live = e0 + tid < nm * G * kC4;
    const int j = (e >= G * kC4 || !f0) ? 1 : 0;  // published run of this item
    const int32_t ej = e - (e >= G * kC4 ? G * kC4 : 0);
    const int32_t g = ej / kC4, c4 = ej - g * kC4;
    const int32_t S0 = j ? p1S0 : p0S0, S1 = j ? p1S1 : p0S1;
    const int32_t bh = j ? p1bh : p0bh, b = bh & 0xFFFF, kvh = bh >> 16;
    const bool device_scope = (j ? f1 : f0) == 2;
    const int32_t la = P.la[j], n = P.n[j];
    // Piece slot of contributor i: the first holds the segment's start
    // (slot 1 of its workgroup), every later one began before its share.
    auto piece = [&](int32_t i) {
      const int32_t l = Tt >= nwg ? la + i : share_of(S0 + i, Tt, nwg);
      return 2 * l + (i == 0 ? 1 : 0);
    };
    // n is uniform within each group of kC4 lanes (one item of one run), so
    // the loops below are too; the shuffles stay inside the group.  Each
    // lane finds one contributor's piece slot and (max, sum); the slots of
    // the others come by shuffle, so the output loads of a batch need no
    // index arithmetic between them.
    floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
    if (!device_scope) {
      float mx = -3.0e38f;
      for (int32_t i0 = 0; i0 < n; i0 += kC4) {
        const int32_t cn = min(kC4, n - i0);
        const int32_t mine = piece(i0 + min(sub, cn - 1));
        const f32x2_t ml = __builtin_bit_cast(
            f32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rml, (mine * G + g) * 8, 0, 0));
        constexpr int kBatch = PA_DECODE_MERGE_BATCH;  // output loads in flight per lane
        for (int32_t u0 = 0; u0 < cn; u0 += kBatch) {
          floatx4_t po[kBatch];
#pragma unroll
          for (int u = 0; u < kBatch; ++u) {
            // Unconditional loads (indices past cn repeat the chunk's last),
            // masked afterwards, so every load of the batch is in flight.
            const int32_t ps = __shfl(mine, base + min(u0 + u, cn - 1));
            po[u] = __builtin_bit_cast(floatx4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                      ro, ((ps * G + g) * D + 4 * c4) * 4, 0, 0));
          }
          // The (max, sum) shuffles wait for their load; keep them after the
          // output loads so that one round trip covers both.
          __builtin_amdgcn_sched_barrier(0);
          float pm[kBatch], pl[kBatch];
#pragma unroll
          for (int u = 0; u < kBatch; ++u) {
            const int src = base + min(u0 + u, cn - 1);
            pm[u] = __shfl(ml[0], src);
            pl[u] = __shfl(ml[1], src);
          }
          float cm = mx;
#pragma unroll
          for (int u = 0; u < kBatch; ++u)
            if (u0 + u < cn) cm = fmaxf(cm, pm[u]);
          const float r = __builtin_amdgcn_exp2f(mx - cm);
          acc *= r;
          den *= r;
#pragma unroll
          for (int u = 0; u < kBatch; ++u) {
            const float w = u0 + u < cn ? __builtin_amdgcn_exp2f(pm[u] - cm) : 0.f;
            acc += w * po[u];
            den = fmaf(w, pl[u], den);
          }
          mx = cm;
        }
      }
    } else {
      // Some contributor ran on another XCD than this one: read every
      // piece at device scope, one at a time (a rare path, kept short).
      float mx = -3.0e38f;
      for (int32_t i = 0; i < n; ++i) {
        const int32_t ps = piece(i);
        const f32x2_t ml = __builtin_bit_cast(
            f32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rml, (ps * G + g) * 8, 0, kDeviceScope));
        const floatx4_t o = __builtin_bit_cast(floatx4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                              ro, ((ps * G + g) * D + 4 * c4) * 4, 0,
                                                              kDeviceScope));
        const float cm = fmaxf(mx, ml[0]);
        const float r = __builtin_amdgcn_exp2f(mx - cm), w = __builtin_amdgcn_exp2f(ml[0] - cm);
        acc = acc * r + w * o;
        den = den * r + w * ml[1];
        mx = cm;
      }
    }
    if (live)
      store_out4<E>(a.out, (((int64_t)b * H_kv + kvh) * G + g) * D + 4 * c4, acc * (1.f / den));
  }
}

// ----------------------------------------------------------- host helpers
size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace of pa_decode_noalloc, for callers that cannot allocate (code
// under HIP graph capture, tight serving loops): one array per GPU, held
// until the process ends.  Fixed regions: the arrival counters in the first
// 4 MiB (so no call's pieces ever land where another call's counters are),
// the published pieces after them.  The array starts zero-filled (static
// storage) and every call leaves its counters at zero, so it needs no
// clearing.  All calls on one GPU share it: overlapping calls race.
constexpr size_t kScratchCtrBytes = 4u << 20;
constexpr size_t kScratchBytes = 21u << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of `scratch` on the current device (its host-side name is
// only a stand-in), looked up once per device.
pa_status scratch_pointer(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return pa::fail(PA_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return pa::fail(PA_ERR_UNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
  std::call_once(g_scratch_once[dev], [dev] {
    g_scratch_err[dev] = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
  });
  if (g_scratch_err[dev] != hipSuccess)
    return pa::fail(PA_ERR_DEVICE, "hipGetSymbolAddress(scratch): %s",
                    hipGetErrorString(g_scratch_err[dev]));
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

struct WorkspaceLayout {
  size_t o_off, ml_off, pieces_end, ctr_off, total;
};

// The published pieces first (their size depends on the head shape only),
// then the arrival counters (the part that must be zero, one per (KV head,
// sequence)).  Calls of one head shape with fewer sequences use a prefix of
// the counters, so a workspace serves every batch size up to the one it was
// sized for without a new zero fill.
WorkspaceLayout workspace_layout(const pa_cache_desc* d, int32_t H_q, int32_t B) {
  const size_t G = H_q / d->num_kv_heads;
  const size_t slots = 2 * (size_t)kMaxWGs;
  WorkspaceLayout w;
  w.o_off = 0;
  w.ml_off = align_up(slots * G * d->head_dim * sizeof(float), 256);
  w.pieces_end = w.ml_off + align_up(slots * G * 2 * sizeof(float), 256);
  w.ctr_off = w.pieces_end;
  w.total = w.ctr_off + align_up((size_t)B * d->num_kv_heads * sizeof(uint64_t), 256);
  return w;
}

// Tiles per batch.  fp32 pools with large query groups hold G*D/16 output
// floats per lane in registers, which leaves room for one tile per batch.
template <bool k16, int D, int GP, bool kAppend>
constexpr int kNbuf = k16 ? (GP >= 8 ? 2 : (kAppend ? PA_DECODE_NB_APPEND : PA_DECODE_NB_BF16))
                          : (GP * D >= 8 * 64 ? 1 : 2);

template <int D, int GP>
size_t lds_bytes(int32_t B) {
  return sizeof(LdsPieces<D, GP>) + (size_t)(2 * B + 1 + kNW) * sizeof(int32_t);
}

template <int E, int D, int GP>
pa_status launch(const DecodeArgs& a, int wgs, hipStream_t s) {
  constexpr int NB = kNbuf<(E != 0), D, GP, false>, NBA = kNbuf<(E != 0), D, GP, true>;
  // K/V loads non-temporal unless the caller expects shared blocks.
  const bool nt = pa::tuning(PA_TUNE_DECODE_KV_CACHED) == 0;
  auto pick = [&](auto kNTc) {
    constexpr bool kNT = decltype(kNTc)::value;
    return a.new_k ? (a.log2_bs >= 4 ? decode_kernel<E, D, GP, NBA, false, true, kNT>
                                     : decode_kernel<E, D, GP, NBA, true, true, kNT>)
                   : (a.log2_bs >= 4 ? decode_kernel<E, D, GP, NB, false, false, kNT>
                                     : decode_kernel<E, D, GP, NB, true, false, kNT>);
  };
  auto kern = nt ? pick(std::true_type{}) : pick(std::false_type{});
  const size_t lds = lds_bytes<D, GP>(a.B);
  if (lds > kMaxLds)
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_decode: %d sequences need %zu bytes of LDS (> %zu)",
                    a.B, lds, kMaxLds);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess)
      return pa::fail(PA_ERR_DEVICE, "pa_decode: LDS attribute: %s", hipGetErrorString(e));
  }
  hipLaunchKernelGGL(kern, dim3(wgs), dim3(kWG), lds, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pa::fail(PA_ERR_DEVICE, "pa_decode: %s", hipGetErrorString(e));
  return PA_OK;
}

template <int E, int D>
pa_status dispatch_g(const DecodeArgs& a, int wgs, hipStream_t s) {
  if (a.G <= 1) return launch<E, D, 1>(a, wgs, s);
  if (a.G <= 2) return launch<E, D, 2>(a, wgs, s);
  if (a.G <= 4) return launch<E, D, 4>(a, wgs, s);
  if (a.G <= 8) return launch<E, D, 8>(a, wgs, s);
  return launch<E, D, 16>(a, wgs, s);
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
  *bytes = workspace_layout(desc, num_q_heads, num_seqs).total;
  return PA_OK;
}

}  // extern "C"

namespace {

// Checks the arguments (all but the workspace) and launches the decode
// with the given workspace parts.
pa_status decode_launch(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                        const int32_t* context_lens, int32_t num_seqs, int32_t block_size,
                        float scale, void* out, int32_t num_q_heads, const pa_cache_desc* desc,
                        float* ws_o, float* ws_ml, uint64_t* counters, void* stream,
                        const void* new_k = nullptr, const void* new_v = nullptr) {
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
  if (desc->num_kv_heads > kMaxKvHeads)
    return pa::fail(PA_ERR_UNSUPPORTED, "num_kv_heads %d > %d", desc->num_kv_heads, kMaxKvHeads);
  const int64_t len_cap = (int64_t)max_blocks_per_seq * block_size;
  if (len_cap > INT32_MAX)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "max_blocks_per_seq * block_size overflows int32");
  // Flat tile indices (KV head, sequence, tile) must fit in int32.
  if ((int64_t)num_seqs * ((len_cap + kTile - 1) / kTile) * desc->num_kv_heads >= (1ll << 31))
    return pa::fail(PA_ERR_UNSUPPORTED, "num_seqs * tiles per sequence * KV heads >= 2^31");
  if (!std::isfinite(scale)) return pa::fail(PA_ERR_INVALID_ARGUMENT, "scale is not finite");
  if (num_seqs == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out || !ws_o || !ws_ml ||
      !counters)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (!pa::aligned(q, 16) || !pa::aligned(k_cache, 16) || !pa::aligned(v_cache, 16) ||
      !pa::aligned(out, 16) || !pa::aligned(block_tables, 4) || !pa::aligned(context_lens, 4))
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "misaligned pointer");
  const int32_t tuned = pa::tuning(PA_TUNE_DECODE_WORKGROUPS);
  const int wgs = tuned >= 1 && tuned <= kMaxWGs ? tuned : kDefaultWGs;
  DecodeArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.tables = block_tables;
  a.lens = context_lens;
  a.out = out;
  a.counters = counters;
  a.ws_o = ws_o;
  a.ws_ml = ws_ml;
  a.new_k = new_k;
  a.new_v = new_v;
  a.B = num_seqs;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = desc->num_blocks;
  a.H_kv = desc->num_kv_heads;
  a.G = num_q_heads / desc->num_kv_heads;
  a.log2_bs = pa::ilog2_exact(block_size);
  a.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  hipStream_t s = (hipStream_t)stream;
  const bool d128 = desc->head_dim == 128;
  switch (desc->dtype) {
    case PA_BF16: return d128 ? dispatch_g<1, 128>(a, wgs, s) : dispatch_g<1, 64>(a, wgs, s);
    case PA_F16: return d128 ? dispatch_g<2, 128>(a, wgs, s) : dispatch_g<2, 64>(a, wgs, s);
    default: return d128 ? dispatch_g<0, 128>(a, wgs, s) : dispatch_g<0, 64>(a, wgs, s);
  }
}

}  // namespace

extern "C" {

pa_status pa_decode(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t num_seqs, int32_t block_size,
                    float scale, void* out, int32_t num_q_heads, const pa_cache_desc* desc,
                    void* workspace, size_t workspace_bytes, void* stream) {
  pa_status st = pa_supported(desc, num_q_heads);
  if (st != PA_OK) return st;
  // The workspace is checked here; every other argument (and a NULL
  // workspace, as a NULL pointer) by decode_launch, in the header's order.
  char* ws = reinterpret_cast<char*>(workspace);
  WorkspaceLayout wl{};
  if (num_seqs > 0 && num_seqs <= kMaxSeqs && ws) {
    if (!pa::aligned(workspace, 256))
      return pa::fail(PA_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
    wl = workspace_layout(desc, num_q_heads, num_seqs);
    if (workspace_bytes < wl.total)
      return pa::fail(PA_ERR_INVALID_ARGUMENT, "workspace %zu bytes < %zu needed",
                      workspace_bytes, wl.total);
  }
  return decode_launch(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, block_size, scale, out, num_q_heads, desc,
                       ws ? reinterpret_cast<float*>(ws + wl.o_off) : nullptr,
                       ws ? reinterpret_cast<float*>(ws + wl.ml_off) : nullptr,
                       ws ? reinterpret_cast<uint64_t*>(ws + wl.ctr_off) : nullptr, stream);
}

pa_status pa_decode_append(const void* q, const void* new_k, const void* new_v, void* k_cache,
                           void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t num_seqs, int32_t block_size,
                           float scale, void* out, int32_t num_q_heads, const pa_cache_desc* desc,
                           void* workspace, size_t workspace_bytes, void* stream) {
  pa_status st = pa_supported(desc, num_q_heads);
  if (st != PA_OK) return st;
  if (num_seqs > 0 && (!new_k || !new_v))
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (!pa::aligned(new_k, 16) || !pa::aligned(new_v, 16))
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "misaligned pointer");
  char* ws = reinterpret_cast<char*>(workspace);
  WorkspaceLayout wl{};
  if (num_seqs > 0 && num_seqs <= kMaxSeqs && ws) {
    if (!pa::aligned(workspace, 256))
      return pa::fail(PA_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
    wl = workspace_layout(desc, num_q_heads, num_seqs);
    if (workspace_bytes < wl.total)
      return pa::fail(PA_ERR_INVALID_ARGUMENT, "workspace %zu bytes < %zu needed",
                      workspace_bytes, wl.total);
  }
  return decode_launch(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, block_size, scale, out, num_q_heads, desc,
                       ws ? reinterpret_cast<float*>(ws + wl.o_off) : nullptr,
                       ws ? reinterpret_cast<float*>(ws + wl.ml_off) : nullptr,
                       ws ? reinterpret_cast<uint64_t*>(ws + wl.ctr_off) : nullptr, stream,
                       num_seqs > 0 ? new_k : nullptr, num_seqs > 0 ? new_v : nullptr);
}

pa_status pa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t num_seqs, int32_t block_size,
                            float scale, void* out, int32_t num_q_heads, const pa_cache_desc* desc,
                            void* stream) {
  pa_status st = pa_supported(desc, num_q_heads);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_seqs > kMaxSeqs)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "num_seqs %d outside [0, %d]", num_seqs, kMaxSeqs);
  // The array's fixed regions: counters in [0, 4 MiB), pieces after.
  const WorkspaceLayout wl = workspace_layout(desc, num_q_heads, num_seqs);
  const size_t ctr_bytes = wl.total - wl.ctr_off;
  if (ctr_bytes > kScratchCtrBytes || wl.pieces_end > kScratchBytes - kScratchCtrBytes)
    return pa::fail(PA_ERR_UNSUPPORTED,
                    "pa_decode_noalloc: this shape needs %zu bytes of counters (at most %zu) and "
                    "%zu bytes of partial results (at most %zu) in its %zu-byte device array "
                    "(use pa_decode with a workspace)",
                    ctr_bytes, kScratchCtrBytes, wl.pieces_end, kScratchBytes - kScratchCtrBytes,
                    kScratchBytes);
  void* base = nullptr;
  if (num_seqs > 0) {
    st = scratch_pointer(&base);
    if (st != PA_OK) return st;
  }
  char* ws = reinterpret_cast<char*>(base);
  char* pieces = ws ? ws + kScratchCtrBytes : nullptr;
  return decode_launch(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, block_size, scale, out, num_q_heads, desc,
                       reinterpret_cast<float*>(pieces ? pieces + wl.o_off : nullptr),
                       reinterpret_cast<float*>(pieces ? pieces + wl.ml_off : nullptr),
                       reinterpret_cast<uint64_t*>(ws), stream);
}

}  // extern "C"
