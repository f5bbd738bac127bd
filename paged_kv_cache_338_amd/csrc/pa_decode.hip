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
//    order (b, KV head, tile).  Wave w of the W waves of the grid takes the
//    equal share [T*w/W, T*(w+1)/W) of the T tiles, so every wave streams
//    the same number of K/V bytes whatever the length mix, and no wave ever
//    waits for another.
//  * Each workgroup first copies the context lengths into LDS with their
//    prefix sums over sequences, so its waves see one consistent snapshot.
//  * Blocks of >= 16 tokens: a wave walks its share as batches of up to
//    NBUF tiles; a batch holds the rest of one segment and, if that segment
//    ends inside it, the start of the next, so crossing a segment boundary
//    costs no extra round trip.  The block ids of the share are fetched 64
//    tiles at a time by one vector load (lane i: tile i) and read with
//    v_readlane a batch ahead; each batch issues its segments' query rows
//    and all its tile loads before the first use.  Smaller blocks: one
//    pipelined piece per segment, block ids gathered per lane.
//  * A segment wholly inside the share is written out by the wave; a piece
//    of a segment cut by a share boundary leaves its online-softmax state
//    (max, sum, unnormalised output) as a partial in the workspace.
//  * A second, small kernel merges the partials of each cut segment (the
//    wave that holds a segment's first tile writes the segment's record), so
//    there is no cross-wave synchronisation inside the decode kernel: on
//    this part, publishing data to other workgroups inside one kernel costs
//    far more (an L2 writeback per release) than a second launch.
//  * Per tile (bf16 pools): the K rows of the 16 tokens are the A operand of
//    a v_mfma_f32_16x16x32_bf16 chain whose B operand is the KV head's G
//    query rows, so the logits of head g and token 4j+r land in lane 16j+g,
//    register r.  The probabilities, rounded to bf16, are the A operand of
//    a v_mfma_f32_16x16x16_bf16 chain against the V rows (D/16 output
//    column blocks) and against a ones operand (the softmax sums), so the
//    output and its normaliser accumulate in MFMA registers.
//    fp32 pools use v_mfma_f32_16x16x4_f32 for the logits and the VALU for
//    P*V, with the probabilities broadcast by DPP.
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
#include <cstdlib>
#include <type_traits>

#include "pa_attn_tile.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace {

using pa::bf16x8_t;
using pa::f32x2_t;
using pa::floatx4_t;
using pa::Geometry;
using pa::issue_tile;
using pa::issue_tile_small;
using pa::kTile;
using pa::kWave;
using pa::MfmaState;
using pa::s16x4_t;
using pa::TileRegs;
using pa::u32x4_t;
using pa::uni;
using pa::uniform_ptr;
constexpr int kMaxWaves = 4096;   // the workspace holds partials for this many waves
constexpr int kDefaultWGs = 256;  // workgroups of the decode grid
constexpr int kMaxSeqs = 8192;    // lengths snapshot in LDS
constexpr int kRecInts = 8;       // ints per segment record
constexpr int kMergeWG = 256;     // threads of the partial-merge kernel
constexpr size_t kMaxLds = 160 * 1024;
#ifndef PA_DECODE_NW
#define PA_DECODE_NW 4  // waves per workgroup
#endif
#ifndef PA_DECODE_OCC_STREAM
#define PA_DECODE_OCC_STREAM 2  // waves per SIMD the streamed bf16 path's registers must allow
#endif
#ifndef PA_DECODE_OCC
#define PA_DECODE_OCC 2  // waves per SIMD the register budget must allow
#endif
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
  float* ws_o;       // [2 * kMaxWaves][G][D] unnormalised partial outputs
  float* ws_m;       // [2 * kMaxWaves][G] running max (log2 units)
  float* ws_l;       // [2 * kMaxWaves][G] sum of exp2(x - max)
  int32_t* records;  // [B * H_kv][kRecInts] per segment: cut? and its contributors
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
  s.nt = max(uni(PB[s.b + 1]) - pb, 1);
  s.kvh = min((f - pb * H_kv) / s.nt, H_kv - 1);
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
// units) that holds unit f, for 0 <= f < T.
__device__ __forceinline__ int32_t share_of(int32_t f, int32_t T, int32_t W) {
  return static_cast<int32_t>((((int64_t)f + 1) * W - 1) / T);
}

template <int E>
__device__ __forceinline__ void store_out(void* out, int64_t i, float x) {
  if constexpr (E != 0) reinterpret_cast<uint16_t*>(out)[i] = pa::round16<E>(x);
  else reinterpret_cast<float*>(out)[i] = x;
}

template <int E, int D, int GP, int kNW, int NBUF, bool kSmall>
__global__ void __launch_bounds__(kNW * kWave)
__attribute__((amdgpu_waves_per_eu(kSmall ? (((E != 0) || GP * D < 16 * 128) ? PA_DECODE_OCC : 1)
                                          : ((E != 0) ? PA_DECODE_OCC_STREAM : 1))))
decode_kernel(DecodeArgs a) {
  constexpr bool BF16 = E != 0;  // 16-bit pools (bf16 or fp16)
  using Geo = Geometry<BF16, D>;
  constexpr int kWG = kNW * kWave;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), v = tid >> 6;
  const int jr = lane >> 4, c16 = lane & 15;
  const int32_t wg = blockIdx.x, nwg = gridDim.x;
  const int32_t B = a.B, H_kv = a.H_kv, G = a.G, H_q = H_kv * G;

  // LDS: the lengths snapshot and its prefix sums.
  int32_t* PB = reinterpret_cast<int32_t*>(smem);  // [B + 1]
  int32_t* Ls = PB + B + 1;                        // [B]
  int32_t* misc = Ls + B;                          // [kNW]

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

  const int32_t Tt = uni(PB[B]) * H_kv;  // flat tiles (host bounds it below 2^31)

  // Sequences with no context get a zero row (workgroup b % W writes it).
  for (int32_t b = wg; b < B; b += nwg) {
    if (Ls[b] == 0) {
      for (int32_t e = tid; e < H_q * D; e += kWG)
        store_out<E>(a.out, (int64_t)b * H_q * D + e, 0.f);
      for (int32_t h = tid; h < H_kv; h += kWG) a.records[(b * H_kv + h) * kRecInts] = 0;
    }
  }
  // ---- this wave's share [G0, G1): wave wv of Wt, the equal share
  // [T*wv/Wt, T*(wv+1)/Wt) of the flat tiles.
  const int32_t Wt = nwg * kNW, wv = wg * kNW + v;
  // floor(Tt * w / Wt) in 32-bit arithmetic: Tt = qt * Wt + rt with rt < Wt
  // <= 4096, so rt * w < 2^24 (64-bit division would cost hundreds of
  // instructions on the critical path of every wave).
  const uint32_t qt = static_cast<uint32_t>(Tt) / static_cast<uint32_t>(Wt);
  const uint32_t rt = static_cast<uint32_t>(Tt) - qt * static_cast<uint32_t>(Wt);
  auto bound = [&](uint32_t w) {
    return static_cast<int32_t>(qt * w + rt * w / static_cast<uint32_t>(Wt));
  };
  const int32_t G0 = uni(bound(wv)), G1 = uni(bound(wv + 1));
  const int log2_bs = a.log2_bs;
  const int nbt = log2_bs >= 4 ? 1 : (kTile >> log2_bs);  // table lanes per tile
  const int tpc_log = log2_bs >= 4 ? 6 : 2 + log2_bs;       // log2(tiles per table chunk)

  using State = std::conditional_t<BF16, MfmaState<D>, WaveState<false, D, GP>>;
  // Finishes segment s after its last tile in this share.  A segment wholly
  // inside the share is written out; a cut piece leaves (max, sum,
  // unnormalised output) in partial slot 2*wv + 0 if the segment began
  // before the share, else 2*wv + 1.
  auto finish = [&](const State& st, const Seg s) {
    const bool whole = s.S0 >= G0 && s.S1 <= G1;
    const int32_t pslot = 2 * wv + (s.S0 < G0 ? 0 : 1);
    float* slot = a.ws_o + (int64_t)pslot * G * D;
    if (s.S0 >= G0 && lane == 0) {
      // This wave holds the segment's first tile: it writes the segment's
      // record for the merge kernel (cut or not, tile range, decomposition).
      int32_t* rec = a.records + (s.b * H_kv + s.kvh) * kRecInts;
      rec[0] = whole ? 0 : 1;
      rec[1] = s.S0;
      rec[2] = s.S1;
      rec[3] = Tt;
      rec[4] = Wt;
      rec[5] = wv;
    }
    if constexpr (BF16) {
      // ---- finish the piece: sums over the 4 rows; the accumulators
      // already hold whole tiles (lane 16j + c, register r: head 4j + r).
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
            for (int i = 0; i < kBlk / 2; ++i) {
              pk[i] = pa::pack2<E>(st.acc[2 * i][q] * inv, st.acc[2 * i + 1][q] * inv);
            }
            char* dst = reinterpret_cast<char*>(a.out) +
                        ((((int64_t)s.b * H_kv + s.kvh) * G + g) * D + kBlk * c16) * 2;
            if constexpr (kBlk == 8) *reinterpret_cast<u32x4_t*>(dst) = u32x4_t{pk[0], pk[1], pk[2], pk[3]};
            else *reinterpret_cast<uint2*>(dst) = uint2{pk[0], pk[1]};
          } else {
            float* dst = slot + g * D + kBlk * c16;
#pragma unroll
            for (int i = 0; i < kBlk; ++i) dst[i] = st.acc[i][q];
          }
        }
        if (!whole && c16 == 0 && g < G) a.ws_l[pslot * G + g] = lg;
      });
      if (!whole && lane < G) a.ws_m[pslot * G + lane] = st.ref;
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
        for (int c = 0; c < Geo::kCols; ++c) {
          o[c] = pa::rows_sum(st.o[g][c] * f);
        }
        if (g < G && (g & 3) == jr) {
          if (whole) {
            const int64_t base = (((int64_t)s.b * H_kv + s.kvh) * G + g) * D + c16 * Geo::kCols;
#pragma unroll
            for (int c = 0; c < Geo::kCols; ++c) store_out<E>(a.out, base + c, o[c] * inv);
          } else {
#pragma unroll
            for (int c = 0; c < Geo::kCols; ++c) slot[g * D + c16 * Geo::kCols + c] = o[c];
          }
        }
      });
      if (!whole && lane < G) {
        a.ws_m[pslot * G + lane] = M;
        a.ws_l[pslot * G + lane] = lt;
      }
    }
  };

  if (G0 < G1) {
    State st;
    st.reset();
    if constexpr (!kSmall) {
      // ---- the share as a stream of batches of up to NBUF tiles.  A batch
      // holds the remaining tiles of one segment A and, if A ends inside
      // it, the first tiles of the next segment B, so a share that crosses
      // a segment boundary costs no extra round trip.  The block ids of the
      // next batch are fetched (scalar loads; the table is read-only during
      // the kernel) while the current batch is consumed, and the query rows
      // of A and B are loaded with the batch's tiles.
      struct Batch {
        Seg A, B;
        int32_t fa;      // flat index of the batch's first tile (in A)
        int32_t nA, n;   // tiles of A; tiles in all (the rest are B's)
        bool endA, endB; // the segment's last tile in this share is here
      };
      Seg cs = seg_containing(PB, Ls, B, H_kv, G0);
      int32_t f = G0;  // next flat tile of the share
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
          seg_advance(cs, PB, Ls, B, H_kv);
          if (bt.nA < NBUF && cs.S0 == f) {
            bt.B = cs;
            const int32_t limB = min(cs.S1, G1);
            const int32_t nB = min(NBUF - bt.nA, limB - f);
            bt.endB = f + nB == limB;
            f += nB;
            bt.n += nB;
            if (f == cs.S1 && f < G1) seg_advance(cs, PB, Ls, B, H_kv);
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
      // Block ids of the share, 64 tiles at a time: lane i of chunk c holds
      // the physical block of flat tile G0 + 64c + i (clamped to the share),
      // found by a per-lane search of the lengths snapshot and one vector
      // load from the table, so batches read their block ids from registers
      // and the table is never on a batch's critical path.
      // Indices are clamped into the table so that no snapshot, however
      // inconsistent, can send a read outside it.
      auto chunk_phys = [&](int32_t c) -> int32_t {
        const int32_t fl = min(G0 + 64 * c + lane, G1 - 1);
        const int32_t b = find_seq(PB, B, H_kv, fl);
        const int32_t pb = PB[b];
        const int32_t nt = max(PB[b + 1] - pb, 1);
        const int32_t r = fl - pb * H_kv;
        const int32_t t = r - (r / nt) * nt;
        const int32_t e = min(max((t * kTile) >> log2_bs, 0), a.max_blocks - 1);
        return a.tables[(int64_t)b * a.max_blocks + e];
      };
      int32_t cbase = G0;  // flat tile of lane 0 of chunk `cur`
      int32_t cur = chunk_phys(0), nxt = 0;
      if (G1 - G0 > 64) nxt = chunk_phys(1);  // read only by shares of more than 64 tiles
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
          issue_tile<BF16, D>(buf[u], a.pool(), ph[u], t, kvh, lane, u < bt.n);
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
      // ---- blocks smaller than a tile: the share as pieces, one per
      // segment, each a pipelined loop over its tiles.
      Seg s = seg_containing(PB, Ls, B, H_kv, G0);
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
          issue_tile_small<BF16, D>(r, a.pool(), dA, jj - (c << tpc_log), t0 + jj, s.kvh, s.L, nbt,
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
        finish(st, s);
        if (s.S1 >= G1) break;
        st.reset();
        seg_advance(s, PB, Ls, B, H_kv);
      }
    }
  }
}

// Merges the partials of segment blockIdx.x (sequence blockIdx.x / H_kv,
// KV head blockIdx.x % H_kv) for query head blockIdx.y of the group, if the
// decode kernel's record says the segment was cut.  The contributors are the
// waves whose shares meet the segment: consecutive ones from the wave wa
// holding its first tile when every share is non-empty (T >= W), else one
// share per tile.  The first contributor's partial is in slot 2w + 1, every
// later one in slot 2w.  Thread t takes the 4-column group t % (D/4) of the
// head's row for the contributors congruent to t / (D/4); the slices'
// (max, sum, output) are then combined through LDS, so the dependent-load
// depth is n / (number of slices), not n.
template <int E, int D>
__global__ void __launch_bounds__(kMergeWG)
merge_kernel(DecodeArgs a) {
  constexpr int kCols = D / 4;
  constexpr int kSlices = kMergeWG / kCols;
  constexpr int kBatch = 8;  // contributors per thread in flight
  __shared__ floatx4_t s_acc[kSlices][kCols];
  __shared__ float s_mx[kSlices], s_den[kSlices];
  const int32_t* rec = a.records + blockIdx.x * kRecInts;
  if (rec[0] == 0) return;
  const int32_t G = a.G, g = blockIdx.y;
  const int32_t b = blockIdx.x / a.H_kv, kvh = blockIdx.x % a.H_kv;
  const int32_t S0 = rec[1], S1 = rec[2], Tt = rec[3], W = rec[4], wa = rec[5];
  // With one tile per non-empty share (T < W <= kMaxWaves), the share of
  // tile f is ((f + 1) W - 1) / T, small enough for 32-bit arithmetic.
  const int32_t n = Tt >= W ? share_of(S1 - 1, Tt, W) - wa + 1 : S1 - S0;
  auto slot_of = [&](int32_t i) {
    const int32_t w = Tt >= W ? wa + i : ((S0 + i + 1) * W - 1) / Tt;
    return 2 * w + (i == 0 ? 1 : 0);
  };
  const int col = threadIdx.x % kCols, k = threadIdx.x / kCols;
  float mx = -3.0e38f, den = 0.f;
  floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int32_t i0 = k; i0 < n; i0 += kSlices * kBatch) {
    // Unconditional loads (indices past n repeat contributor i0), masked
    // afterwards, so every load of the batch is in flight at once.
    float pm[kBatch], pl[kBatch];
    floatx4_t po[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int32_t i = i0 + u * kSlices;
      const int32_t slot = slot_of(i < n ? i : i0);
      pm[u] = a.ws_m[slot * G + g];
      pl[u] = a.ws_l[slot * G + g];
      po[u] = *reinterpret_cast<const floatx4_t*>(a.ws_o + ((int64_t)slot * G + g) * D + 4 * col);
    }
    float cm = mx;
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (i0 + u * kSlices < n) cm = fmaxf(cm, pm[u]);
    const float r = __builtin_amdgcn_exp2f(mx - cm);
    acc *= r;
    den *= r;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float f = i0 + u * kSlices < n ? __builtin_amdgcn_exp2f(pm[u] - cm) : 0.f;
      acc += f * po[u];
      den = fmaf(f, pl[u], den);
    }
    mx = cm;
  }
  s_acc[k][col] = acc;
  if (col == 0) {
    s_mx[k] = mx;
    s_den[k] = den;
  }
  __syncthreads();
  if (k != 0) return;
  float M = s_mx[0];
#pragma unroll
  for (int j = 1; j < kSlices; ++j) M = fmaxf(M, s_mx[j]);
  floatx4_t o = {0.f, 0.f, 0.f, 0.f};
  float l = 0.f;
#pragma unroll
  for (int j = 0; j < kSlices; ++j) {
    const float f = __builtin_amdgcn_exp2f(s_mx[j] - M);  // 0 for an empty slice
    o += f * s_acc[j][col];
    l = fmaf(f, s_den[j], l);
  }
  const float inv = 1.f / l;
  const int64_t base = (((int64_t)b * a.H_kv + kvh) * G + g) * D + 4 * col;
  if constexpr (E != 0) {
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + base) =
        uint2{pa::pack2<E>(o[0] * inv, o[1] * inv), pa::pack2<E>(o[2] * inv, o[3] * inv)};
  } else {
    *reinterpret_cast<floatx4_t*>(reinterpret_cast<float*>(a.out) + base) = o * inv;
  }
}

// ----------------------------------------------------------- host helpers
int decode_wgs(int nw) {
  // Tuning override (read on every call): PA_DECODE_WGS = workgroups of
  // the decode grid.  Any value gives the same result up to fp32 rounding.
  const char* e = std::getenv("PA_DECODE_WGS");
  const int x = e ? std::atoi(e) : kDefaultWGs;
  return x >= 1 && x * nw <= kMaxWaves ? x : kDefaultWGs;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct WorkspaceLayout {
  size_t rec_off, o_off, m_off, l_off, total;
};

WorkspaceLayout workspace_layout(const pa_cache_desc* d, int32_t H_q, int32_t B) {
  const size_t G = H_q / d->num_kv_heads;
  WorkspaceLayout w;
  w.rec_off = 0;
  w.o_off = align_up((size_t)B * d->num_kv_heads * kRecInts * sizeof(int32_t), 256);
  w.m_off = w.o_off + align_up((size_t)2 * kMaxWaves * G * d->head_dim * sizeof(float), 256);
  w.l_off = w.m_off + align_up((size_t)2 * kMaxWaves * G * sizeof(float), 256);
  w.total = w.l_off + align_up((size_t)2 * kMaxWaves * G * sizeof(float), 256);
  return w;
}

// Waves per workgroup and tiles per batch.  Waves are independent, so the
// workgroup size only sets how often the lengths prologue is repeated.
template <bool k16, int D, int GP>
struct Config {
  static constexpr int kNW = PA_DECODE_NW;
  // fp32 pools with large query groups hold G*D/16 output floats per lane
  // in registers, which leaves room for one tile per batch only.
  static constexpr int NBUF =
      k16 ? (GP >= 8 ? 2 : PA_DECODE_NB_BF16) : (GP * D >= 8 * 64 ? 1 : 2);
};

size_t lds_bytes(int nw, int32_t B) { return (size_t)(2 * B + 1 + nw) * sizeof(int32_t); }

template <int E, int D, int GP>
pa_status launch(const DecodeArgs& a, hipStream_t s) {
  using C = Config<(E != 0), D, GP>;
  auto kern = a.log2_bs >= 4 ? decode_kernel<E, D, GP, C::kNW, C::NBUF, false>
                             : decode_kernel<E, D, GP, C::kNW, C::NBUF, true>;
  const size_t lds = lds_bytes(C::kNW, a.B);
  if (lds > kMaxLds)
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_decode: %d sequences need %zu bytes of LDS (> %zu)",
                    a.B, lds, kMaxLds);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess)
      return pa::fail(PA_ERR_DEVICE, "pa_decode: LDS attribute: %s", hipGetErrorString(e));
  }
  const int wgs = decode_wgs(C::kNW);
  hipLaunchKernelGGL(kern, dim3(wgs), dim3(C::kNW * kWave), lds, s, a);
  hipLaunchKernelGGL((merge_kernel<E, D>), dim3(a.B * a.H_kv, a.G), dim3(kMergeWG), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pa::fail(PA_ERR_DEVICE, "pa_decode: %s", hipGetErrorString(e));
  return PA_OK;
}

template <int E, int D>
pa_status dispatch_g(const DecodeArgs& a, hipStream_t s) {
  if (a.G <= 1) return launch<E, D, 1>(a, s);
  if (a.G <= 2) return launch<E, D, 2>(a, s);
  if (a.G <= 4) return launch<E, D, 4>(a, s);
  if (a.G <= 8) return launch<E, D, 8>(a, s);
  return launch<E, D, 16>(a, s);
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
  // Segment records and flat tile indices (sequence, KV head, tile) must fit
  // in int32.
  if ((int64_t)num_seqs * desc->num_kv_heads * kRecInts >= (1ll << 31))
    return pa::fail(PA_ERR_UNSUPPORTED, "num_seqs * KV heads too large");
  if ((int64_t)num_seqs * ((len_cap + kTile - 1) / kTile) * desc->num_kv_heads >= (1ll << 31))
    return pa::fail(PA_ERR_UNSUPPORTED, "num_seqs * tiles per sequence * KV heads >= 2^31");
  if (!std::isfinite(scale)) return pa::fail(PA_ERR_INVALID_ARGUMENT, "scale is not finite");
  if (num_seqs == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out || !workspace)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (!pa::aligned(workspace, 256))
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
  if (!pa::aligned(q, 16) || !pa::aligned(k_cache, 16) || !pa::aligned(v_cache, 16) ||
      !pa::aligned(out, 16) || !pa::aligned(block_tables, 4) || !pa::aligned(context_lens, 4))
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "misaligned pointer");
  const WorkspaceLayout wl = workspace_layout(desc, num_q_heads, num_seqs);
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
  const bool d128 = desc->head_dim == 128;
  switch (desc->dtype) {
    case PA_BF16: return d128 ? dispatch_g<1, 128>(a, s) : dispatch_g<1, 64>(a, s);
    case PA_F16: return d128 ? dispatch_g<2, 128>(a, s) : dispatch_g<2, 64>(a, s);
    default: return d128 ? dispatch_g<0, 128>(a, s) : dispatch_g<0, 64>(a, s);
  }
}

}  // extern "C"
