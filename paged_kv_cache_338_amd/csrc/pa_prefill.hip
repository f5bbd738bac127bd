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
// Work decomposition: a workgroup takes one (sequence, KV head, query
// block): 4 waves x R row blocks x 16 rows, a row being one (query token,
// head of the KV head's group) pair, GP heads per token (G rounded up to a
// power of two; rows of heads >= G are padding).  Items go longest first:
// sequences by length (for batches of up to 256), each one's query blocks
// from the last.  The workgroup walks the keys of its causal range in tiles
// of 32: the 256 threads gather a tile's K and V rows through the block
// table into registers (tiles ahead, with the table entries read one tile
// earlier still), store them to a double-buffered, padded LDS tile, and
// every wave then computes its rows against it.  So each K/V byte crosses
// the cache hierarchy once per 64 R rows, not once per 16.
//
// Per tile and row block, on the MFMA units (v_mfma_f32_16x16x32, bf16 or
// fp16): S = K Q^T (two 16-key blocks), the lazily rescaled online softmax
// of the decode kernel, then O += P V and l += P 1 with the 32 keys as the
// contraction, V read from LDS by transposing reads straight into the
// operand layout.  Only the tiles that cross a wave's first diagonal mask
// anything; K/V rows past the cache length are loaded as zeros.
//
// pa_prefill_split, for calls with few query blocks: each query block's key
// range is cut into pieces of key tiles, one workgroup per piece, which
// leaves per row (reference maximum, sum, unnormalised output) in a
// workspace; a second kernel merges a block's pieces.
//
// The query rows are MFMA operands in the pool's 16-bit format, so the call
// takes bf16 or fp16 pools.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>

#include "pa_attn_tile.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace {

using pa::f32x2_t;
using pa::floatx4_t;
using pa::kWave;
using pa::u32x4_t;
using pa::uni;

constexpr int kNW = 4;          // waves per workgroup
constexpr int kThreads = kNW * kWave;
constexpr int kMaxSeqs = 8192;  // query starts and lengths snapshot in LDS
constexpr int kKT = 32;         // keys per LDS tile
constexpr int kOcc = 2;         // waves per SIMD the registers are sized for
#ifndef PA_PREFILL_PD1
#define PA_PREFILL_PD1 4  // tiles of loads in flight with one row block per wave
#endif
#ifndef PA_PREFILL_ROW_PAD
#define PA_PREFILL_ROW_PAD 32  // bytes of padding per LDS row (build-time tuning knob)
#endif
#ifndef PA_PREFILL_PD2
#define PA_PREFILL_PD2 2  // ... with two (its registers hold two)
#endif
// Row blocks per wave: 2 normally, 1 when that leaves too few workgroups
// to fill the chip (measured on the Llama-3-8B shape: R = 2 is faster from
// about two workgroups per CU up, R = 1 below).
constexpr int64_t kMinItemsR2 = 512;
// Up to this many sequences, items are taken in the order of the sequences'
// lengths, longest first (each workgroup ranks the lengths in its prologue);
// beyond it, in batch order.
constexpr int kSortMax = 256;
static_assert(kSortMax <= kNW * kWave, "one sequence per thread while ranking");

// Bytes of the LDS header (per-sequence snapshot) in front of the K/V tiles:
// query starts, query counts, prefix sums, wave totals, the processing
// order (up to kSortMax sequences) and, when long items are split along the
// keys, each sequence's number of pieces.
__host__ __device__ constexpr int32_t header_bytes(int32_t B, bool split) {
  return ((3 * B + 1 + kNW + (B <= kSortMax ? B : 0) + (split ? B : 0)) * 4 + 15) & ~15;
}

// Rows of one workgroup's partial state when items are split (one 16-row
// block per wave).
constexpr int kPieceRows = kNW * 16;

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
  // Split items only: key tiles per piece, and per workgroup (piece) and
  // row its unnormalised output [grid][kPieceRows][D] and its reference
  // maximum (log2 units) and sum [grid][kPieceRows][2].
  int32_t key_tiles;
  float* ws_o;
  float* ws_ml;
};

template <int D>
struct TileGeo {
  static constexpr int kRowBytes = D * 2;
  // LDS rows padded by PA_PREFILL_ROW_PAD bytes (a multiple of 16).  With
  // the K rows read 16 bytes per lane and V by transposing reads, 32 bytes
  // is the fastest of 16, 32, 48 and 64 on the worked batch (whole prompts
  // 298 us against 304-305 us).
  static constexpr int kRowLds = kRowBytes + PA_PREFILL_ROW_PAD;
  static constexpr int kMat = kKT * kRowLds;           // one K or V tile in LDS
  static constexpr int kStage = 2 * kMat;              // K then V
  static constexpr int kPPR = kRowBytes / 16;          // 16-byte pieces per row
  static constexpr int kLoads = kKT * kPPR / kThreads; // pieces per thread per matrix
  static constexpr int kDS = D / 32;                   // QK contraction slices
  static constexpr int kBlk = D / 16;                  // output columns per lane
  static_assert(kLoads >= 1 && kKT * kPPR % kThreads == 0, "tile must split over the threads");
};

// ds_read_b64_tr_b16 (gfx950): 64 bits per lane from an LDS address, returned
// transposed within each 16-lane row (lane i gets element i % 4 of the four
// 16-bit values at lane 4e + i / 4's address, e = 0..3).  p must point into
// LDS, 8-byte aligned.
__device__ __forceinline__ uint2 lds_read_tr16(const char* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(uint2, x);
}

// Largest r in [0, B) with P[r] * H <= f (P: exclusive prefix sums in LDS).
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

// One work item: key tiles [t_lo, t_hi) for the query tokens [i0, i1) of
// sequence b (query rows from qs on, nq query tokens, L cache tokens)
// against KV head kvh; piece s of the S pieces of its query block (S = 1
// when items are not split).
struct Item {
  int32_t b, kvh, qs, nq, L, i0, i1, t_lo, t_hi, s, S;
};

// Key tiles a query block sees: keys 0 .. the position of its last token.
__device__ __forceinline__ int32_t block_tiles(int32_t L, int32_t nq, int32_t qb, int32_t QT) {
  return (L - nq + min((qb + 1) * QT, nq) - 1) / kKT + 1;
}

// The workgroup prologue of the attention and merge kernels: the
// per-sequence snapshot in the LDS header, the processing order, and the
// item of workgroup blockIdx.x.  Returns false (for the whole workgroup)
// when blockIdx.x is past the last item.  QT: query tokens per query
// block; kSplit: query blocks are cut into pieces of a.key_tiles key tiles.
template <int QT, bool kSplit>
__device__ bool locate_item(const PrefillArgs& a, char* smem, Item& it) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), v = tid >> 6;
  const int32_t B = a.B, H_kv = a.pool.H_kv;
  const int32_t len_cap = a.max_blocks << a.pool.log2_bs;
  const int32_t kt_per = kSplit ? a.key_tiles : 1;
  // LDS: per sequence the query start and the number of query tokens n_b
  // (clamped to [0, L_b]); the exclusive prefix sums of its items in
  // processing order; for short batches the processing order itself (ORD:
  // rank -> sequence, longest sequence first, so that the items that walk
  // the most key tiles start first and the grid ends on short ones); for
  // split items each sequence's number of pieces.
  const bool sorted = B <= kSortMax;
  int32_t* QS = reinterpret_cast<int32_t*>(smem);  // [B]
  int32_t* NQ = QS + B;                            // [B]
  int32_t* PQ = NQ + B;                            // [B + 1]
  int32_t* misc = PQ + B + 1;                      // [kNW]
  int32_t* ORD = misc + kNW;                       // [B] when sorted
  int32_t* NP = ORD + (sorted ? B : 0);            // [B] when split
  for (int32_t b = tid; b < B; b += kThreads) {
    const int32_t q0 = min(max(a.qstart[b], 0), a.T);
    const int32_t q1 = min(max(a.qstart[b + 1], q0), a.T);
    const int32_t L = min(max(a.lens[b], 0), len_cap);
    const int32_t n = min(q1 - q0, L);
    QS[b] = q0;
    NQ[b] = n;
    PQ[b] = n > 0 ? L : -1;  // ranking key, replaced by the prefix sums below
    if constexpr (kSplit) {
      int32_t np = 0;
      for (int32_t qb = 0; qb * QT < n; ++qb) np += (block_tiles(L, n, qb, QT) + kt_per - 1) / kt_per;
      NP[b] = np;
    }
  }
  __syncthreads();
  if (sorted) {
    // The last query token of a sequence attends to all of its L keys, so
    // its first item walks ceil(L / 32) tiles: rank by L, ties by index.
    int32_t rank = 0;
    if (tid < B) {
      const int32_t key = PQ[tid];
      for (int32_t j = 0; j < B; ++j) {
        const int32_t kj = PQ[j];
        rank += (kj > key || (kj == key && j < tid)) ? 1 : 0;
      }
    }
    __syncthreads();
    if (tid < B) ORD[rank] = tid;
    __syncthreads();
  }
  int32_t carry = 0;
  for (int32_t c = 0; c < B; c += kThreads) {
    const int32_t r = c + tid;
    int32_t nt = 0;
    if (r < B) {
      const int32_t b = sorted ? ORD[r] : r;
      nt = kSplit ? NP[b] : (NQ[b] + QT - 1) / QT;
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
    if (r < B) PQ[r] = pre + incl - nt;
    carry += tot;
    __syncthreads();
  }
  if (tid == 0) PQ[B] = carry;
  __syncthreads();

  // ---- this workgroup's item: sequences in processing order, each one's
  // query blocks longest first; a query block's items are its pieces (in
  // key order) times the KV heads.
  const int32_t items = uni(PQ[B]) * H_kv;
  const int32_t f = blockIdx.x;
  if (f >= items) return false;
  const int32_t rk = uni(find_item_seq(PQ, B, H_kv, f));
  it.b = sorted ? uni(ORD[rk]) : rk;
  int32_t local = f - uni(PQ[rk]) * H_kv;
  it.nq = uni(NQ[it.b]);
  it.qs = uni(QS[it.b]);
  it.L = min(max(a.lens[it.b], 0), len_cap);  // uniform (scalar load)
  int32_t qb = (it.nq + QT - 1) / QT - 1;
  if constexpr (kSplit) {
    int32_t np = (block_tiles(it.L, it.nq, qb, QT) + kt_per - 1) / kt_per;
    while (qb > 0 && local >= np * H_kv) {
      local -= np * H_kv;
      --qb;
      np = (block_tiles(it.L, it.nq, qb, QT) + kt_per - 1) / kt_per;
    }
    it.S = np;
    it.s = local / H_kv;
    it.kvh = local - it.s * H_kv;
    if (it.s >= it.S) return false;  // only if the snapshot disagreed with itself
  } else {
    it.kvh = local % H_kv;
    qb -= local / H_kv;
    it.s = 0;
    it.S = 1;
  }
  it.i0 = qb * QT;
  it.i1 = min(it.i0 + QT, it.nq);
  const int32_t ntiles = block_tiles(it.L, it.nq, qb, QT);
  it.t_lo = kSplit ? it.s * kt_per : 0;
  it.t_hi = kSplit ? min(it.t_lo + kt_per, ntiles) : ntiles;
  return true;
}

template <int E, int D, int GP, int R, bool kSplit>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kOcc, kOcc)))
prefill_kernel(PrefillArgs a) {
  static_assert(!kSplit || R == 1, "split items take one row block per wave");
  using Geo = TileGeo<D>;
  constexpr int kBlk = Geo::kBlk, kDS = Geo::kDS, kLoads = Geo::kLoads;
  constexpr int TP = 16 / GP;          // query tokens per 16-row block
  constexpr int QW = R * TP;           // query tokens per wave
  constexpr int QT = kNW * QW;         // query tokens per workgroup
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), v = tid >> 6;
  const int jr = lane >> 4, c16 = lane & 15;
  const int32_t H_kv = a.pool.H_kv, G = a.G, H_q = H_kv * G;
  const int log2_bs = a.pool.log2_bs;

  Item it;
  if (!locate_item<QT, kSplit>(a, smem, it)) return;
  char* tiles = smem + header_bytes(a.B, kSplit);
  const int32_t b = it.b, kvh = it.kvh, nq = it.nq, L = it.L;
  const int32_t pbase = L - nq;                       // position of query token 0
  const int32_t i0 = it.i0, i1 = it.i1;               // the workgroup's tokens
  const int32_t tlo = it.t_lo, nloc = it.t_hi - it.t_lo;  // its key tiles
  // This wave's tokens [w0, w1) and positions.
  const int32_t w0 = i0 + v * QW, w1 = min(w0 + QW, i1);
  const bool wave_live = w0 < w1;
  const int32_t wp_min = pbase + w0, wp_max = pbase + w1 - 1;

  // Query rows: row block r, lane c16 is row c16 = (token w0 + r*TP + c16/GP,
  // head c16 % GP); padding rows are zero and take the wave's last position
  // as their causal limit.
  // A negative scale is applied as |scale| to the negated query (an exact
  // sign flip in bf16), so that the largest score is the largest logit.
  const float scale = fabsf(a.scale_log2);
  const uint32_t qsign_w = a.scale_log2 < 0.f ? 0x80008000u : 0u;
  const u32x4_t qsign = {qsign_w, qsign_w, qsign_w, qsign_w};
  u32x4_t qf[R][kDS];
  int32_t lim[R];
  {
    const int32_t qs_b = it.qs;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int32_t ti = w0 + r * TP + c16 / GP, g = c16 % GP;
      const bool live = ti < w1 && g < G;
      lim[r] = live ? pbase + ti : wp_max;
      const int64_t row = (int64_t)(qs_b + (live ? ti : 0)) * H_q + kvh * G + (live ? g : 0);
      const char* qp = reinterpret_cast<const char*>(a.q) + row * Geo::kRowBytes + jr * 16;
#pragma unroll
      for (int ds = 0; ds < kDS; ++ds) {
        const u32x4_t x = *reinterpret_cast<const u32x4_t*>(qp + ds * 64);
        qf[r][ds] = live ? (x ^ qsign) : u32x4_t{0, 0, 0, 0};
      }
    }
  }

  // ---- K/V tile gather: thread tid moves row tid / 8 of every tile, its
  // 16-byte column pieces (tid % 8) + 8 h (h < kLoads), of K and of V: one
  // table entry and one address per tile, and 8 lanes store 128
  // contiguous bytes of a row at a time.  Pool rows are numbered in 32 bits
  // (the host bounds num_blocks * H_kv * bs).
  const int32_t* trow = a.tables + (int64_t)b * a.max_blocks;
  const int my_row = tid >> 3, col0 = tid & 7;
  constexpr int kPieceStep = 8 * 16;
  const int32_t bs_mask = (1 << log2_bs) - 1;
  const int32_t rows_per_block = H_kv << log2_bs, kv_row = kvh << log2_bs;
  const char* kbase = reinterpret_cast<const char*>(a.pool.k_cache) + col0 * 16;
  const char* vbase = reinterpret_cast<const char*>(a.pool.v_cache) + col0 * 16;
  const int32_t nb1 = a.pool.num_blocks - 1;
  // Tile indices kt below count from the item's first key tile, tlo.
  auto table_entry = [&](int32_t kt) __attribute__((always_inline)) -> int32_t {
    const int32_t key = min((tlo + kt) * kKT + my_row, L - 1);
    return trow[min(key >> log2_bs, a.max_blocks - 1)];
  };
  // Every lane loads (the row is clamped into the cache), so the number of
  // loads in flight is the same on every path; stash zeroes rows past it.
  auto gather = [&](int32_t kt, int32_t tb, u32x4_t (&kr)[kLoads],
                    u32x4_t (&vr)[kLoads]) __attribute__((always_inline)) {
    const int32_t key = min((tlo + kt) * kKT + my_row, L - 1);
    const uint32_t row = (uint32_t)(min(max(tb, 0), nb1) * rows_per_block + kv_row) +
                         (uint32_t)(key & bs_mask);
    const uint64_t off = (uint64_t)row * Geo::kRowBytes;
#pragma unroll
    for (int h = 0; h < kLoads; ++h) {
      kr[h] = *reinterpret_cast<const u32x4_t*>(kbase + off + h * kPieceStep);
      vr[h] = *reinterpret_cast<const u32x4_t*>(vbase + off + h * kPieceStep);
    }
  };
  const int lds_off = my_row * Geo::kRowLds + col0 * 16;
  auto stash = [&](int32_t kt, int stage, const u32x4_t (&kr)[kLoads],
                   const u32x4_t (&vr)[kLoads]) __attribute__((always_inline)) {
    char* kl = tiles + stage * Geo::kStage + lds_off;
    if ((tlo + kt) * kKT + kKT > L) {  // uniform: the tile reaches past the cache
      const bool in = (tlo + kt) * kKT + my_row < L;
#pragma unroll
      for (int h = 0; h < kLoads; ++h) {
        *reinterpret_cast<u32x4_t*>(kl + h * kPieceStep) = in ? kr[h] : u32x4_t{0, 0, 0, 0};
        *reinterpret_cast<u32x4_t*>(kl + Geo::kMat + h * kPieceStep) = in ? vr[h] : u32x4_t{0, 0, 0, 0};
      }
    } else {
#pragma unroll
      for (int h = 0; h < kLoads; ++h) {
        *reinterpret_cast<u32x4_t*>(kl + h * kPieceStep) = kr[h];
        *reinterpret_cast<u32x4_t*>(kl + Geo::kMat + h * kPieceStep) = vr[h];
      }
    }
  };

  // ---- per-row-block softmax state (the decode kernel's conventions):
  //  ref[r]: lane 16j + c: reference max of row c (log2 units); thr[r] the
  //  raw score above which a logit exceeds ref[r] + 8;
  //  l[r], acc[r][blk]: lane 16j + c, register q: row 4j + q; acc at
  //  column 16 blk + c.
  float ref[R], thr[R];
  floatx4_t l[R];
  floatx4_t acc[R][kBlk];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    ref[r] = -3.0e38f;
    thr[r] = -3.0e38f;
    l[r] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kBlk; ++k) acc[r][k] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  }
  const float inv_scale = scale > 0.f ? 1.f / scale : 0.f;
  constexpr uint32_t k1 = pa::kOnes2<E>;
  const u32x4_t ones = {k1, k1, k1, k1};

  // Raw scores of a tile: s[kb][r], lane 16j + c, register q = key
  // t0 + 16 kb + 4j + q against row c of block r; masked keys are -inf.
  // front also reads the tile's V words (vw) right after the QK MFMAs, so
  // their LDS latency overlaps the softmax.
  floatx4_t s[2][R];
  uint2 vt[kBlk][2];  // V[16 kb + 4j + e][16 blk + c], e = 0..3, as 4 16-bit values
  auto front = [&](int stage, int32_t t0, bool masked) __attribute__((always_inline)) -> bool {
    const char* Kl = tiles + stage * Geo::kStage;
    const char* Vl = Kl + Geo::kMat;
    u32x4_t kf[2][kDS];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ds = 0; ds < kDS; ++ds)
        kf[kb][ds] = *reinterpret_cast<const u32x4_t*>(
            Kl + (kb * 16 + c16) * Geo::kRowLds + ds * 64 + jr * 16);
    __builtin_amdgcn_sched_barrier(0);  // all K reads in flight before the first MFMA
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < R; ++r) s[kb][r] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < kDS; ++ds) {
#pragma unroll
        for (int r = 0; r < R; ++r)
          s[kb][r] = pa::mfma_k32<E>(kf[kb][ds], qf[r][ds], s[kb][r]);
      }
    }
    // V through gfx950's transposing LDS read (ds_read_b64_tr_b16): within
    // each 16-lane row j, lane i receives element i % 4 of the 4 16-bit
    // values that lane 4e + i / 4 points at, e = 0..3.  Lane 16j + s points
    // at key 4j + s / 4, columns 16 blk + 4 (s % 4) .. + 3, so lane 16j + c
    // receives V[4j + e][16 blk + c]: the MFMA operand of column c over the
    // keys 4j .. 4j + 3 (kb = 0) or 16 + 4j .. (kb = 1), in P's key order.
    {
      const char* vsrc = Vl + (4 * jr + (c16 >> 2)) * Geo::kRowLds + (c16 & 3) * 8;
#pragma unroll
      for (int k = 0; k < kBlk; ++k)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          vt[k][kb] = lds_read_tr16(vsrc + kb * 16 * Geo::kRowLds + k * 32);
    }
    if (masked) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (t0 + kb * 16 + 4 * jr + q > lim[r]) s[kb][r][q] = -INFINITY;
    }
    // Any score above its row's threshold: plain compares (no reduction).
    bool hi = false;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int q = 0; q < 4; ++q) hi |= s[kb][r][q] > thr[r];
    return __ballot(hi) != 0;
  };
  // Raises the references to the tile's row maxima (where larger) and
  // rescales l and acc: the only place that touches them outside an MFMA.
  auto rescale = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float m = fmaxf(fmaxf(fmaxf(s[0][r][0], s[0][r][1]), fmaxf(s[0][r][2], s[0][r][3])),
                      fmaxf(fmaxf(s[1][r][0], s[1][r][1]), fmaxf(s[1][r][2], s[1][r][3])));
      m = pa::rows_max(m) * scale;
      const float nref = fmaxf(ref[r], m);
      const float fac = __builtin_amdgcn_exp2f(ref[r] - nref);
      ref[r] = nref;
      thr[r] = (nref + 8.f) * inv_scale;
      pa::static_for<0, 4>([&](auto Q) {
        constexpr int q = decltype(Q)::value;
        const float fr = pa::pick_row_quad<q>(fac, jr);  // row 4j + q
        l[r][q] *= fr;
#pragma unroll
        for (int k = 0; k < kBlk; ++k) acc[r][k][q] *= fr;
      });
    }
  };
  // p = 2^(score * scale - ref) as the 32-deep operand (the lane's keys
  // 4j..4j+3, then 16+4j..16+4j+3), l += P 1, O += P V.
  auto back = [&]() __attribute__((always_inline)) {
    u32x4_t pp[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float nr = -ref[r];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        pp[r][2 * kb] = pa::pack2<E>(__builtin_amdgcn_exp2f(fmaf(s[kb][r][0], scale, nr)),
                                     __builtin_amdgcn_exp2f(fmaf(s[kb][r][1], scale, nr)));
        pp[r][2 * kb + 1] = pa::pack2<E>(__builtin_amdgcn_exp2f(fmaf(s[kb][r][2], scale, nr)),
                                         __builtin_amdgcn_exp2f(fmaf(s[kb][r][3], scale, nr)));
      }
      l[r] = pa::mfma_k32<E>(pp[r], ones, l[r]);
    }
    // For column block blk the lane's operand is V[key][16 blk + c] over its
    // 8 keys, in P's key order, as the transposing reads left it.
#pragma unroll
    for (int k = 0; k < kBlk; ++k) {
      const u32x4_t vb = {vt[k][0].x, vt[k][0].y, vt[k][1].x, vt[k][1].y};
#pragma unroll
      for (int r = 0; r < R; ++r)
        acc[r][k] = pa::mfma_k32<E>(pp[r], vb, acc[r][k]);
    }
  };

  // ---- the key loop, N tiles of loads in flight (N register sets): at tile
  // kt, set kt % N holds tile kt (stored to LDS stage kt % 2, then reloaded
  // with tile kt + N) and the other sets hold tiles kt + 1 .. kt + N - 1.
  // The table entry of a tile is read before the gather of the tile before
  // it, so waiting for it never waits for that gather (loads complete in
  // order).  A tile whose logits exceed a reference leaves the inner loop
  // (after its one barrier, like every tile) to be rescaled and finished
  // outside it, so the hot loop touches the accumulators only through MFMA.
  constexpr int N = R == 1 ? PA_PREFILL_PD1 : PA_PREFILL_PD2;
  static_assert(N >= 2 && N % 2 == 0, "an even number of register sets");
  int32_t tb[2];
  u32x4_t kr[N][kLoads], vr[N][kLoads];
  // Tiles past the last are gathered too (clamped, never used): the loads
  // are unconditional so that the waits stay exact.
  {
    int32_t cur = table_entry(0);
    pa::static_for<0, N>([&](auto J) {
      constexpr int j = decltype(J)::value;
      const int32_t next = table_entry(j + 1);
      gather(j, cur, kr[j], vr[j]);
      cur = next;
    });
    tb[0] = cur;  // tile N's entry
  }
  // One tile: returns true when it must be rescaled (its scores in s).
  auto step = [&](int32_t kt, auto kSet) __attribute__((always_inline)) -> bool {
    constexpr int x = decltype(kSet)::value, p = x & 1;
    stash(kt, p, kr[x], vr[x]);
    tb[1 - p] = table_entry(kt + N + 1);
    gather(kt + N, tb[p], kr[x], vr[x]);
    pa::lds_barrier();
    const int32_t t0 = (tlo + kt) * kKT;
    // Spare tiles past the item's last (kt >= nloc) compute nothing: for a
    // piece of a split query block they are the next piece's keys.
    if (wave_live && kt < nloc && t0 <= wp_max) {
      if (front(p, t0, t0 + kKT - 1 > wp_min)) return true;
      back();
    }
    return false;
  };
  // Tile kt with its set chosen at run time (only after a rescale).
  auto step_any = [&](int32_t kt) __attribute__((always_inline)) -> bool {
    bool r = false;
    pa::static_for<0, N>([&](auto X) {
      if (kt % N == decltype(X)::value) r = step(kt, X);
    });
    return r;
  };
  // Tiles go in groups of N (sets 0 .. N-1), so the register sets keep
  // their registers across iterations; the count is rounded up to a
  // multiple of N (spare last tiles compute nothing), and every wave passes
  // exactly one barrier per tile on every path.
  const int32_t ntot = (nloc + N - 1) / N * N;
  int32_t kt = 0;
  while (true) {
    bool brk = false;
    while (kt % N != 0 && kt < ntot) {  // back from a rescale: realign
      if (step_any(kt)) {
        brk = true;
        break;
      }
      ++kt;
    }
    if (!brk) {
      for (; kt < ntot; kt += N) {
        int u = -1;
        pa::static_for<0, N>([&](auto U) {
          constexpr int x = decltype(U)::value;
          if (u < 0 && step(kt + x, U)) u = x;
        });
        if (u >= 0) {
          kt += u;
          brk = true;
          break;
        }
      }
    }
    if (!brk) break;
    rescale();
    back();
    ++kt;
  }

  // ---- finish: row block r, lane 16j + c, register q holds row 4j + q at
  // columns kBlk * c .. kBlk * c + kBlk - 1; its normaliser is l[r][q].
  if (!wave_live) return;
  if constexpr (kSplit) {
    if (it.S > 1) {
      // A piece of a split query block: per row its reference maximum (the
      // base of the exponentials in acc and l), l and the unnormalised
      // output, for the merge kernel.
      const int64_t base = (int64_t)blockIdx.x * kPieceRows + v * 16;
      pa::static_for<0, 4>([&](auto Q) {
        constexpr int q = decltype(Q)::value;
        const int row = 4 * jr + q;
        const float refq = pa::pick_row_quad<q>(ref[0], jr);  // row 4j + q
        const int32_t ti = w0 + row / GP, g = row % GP;
        if (ti < w1 && g < G) {
          float* o = a.ws_o + (base + row) * D + c16;
#pragma unroll
          for (int k = 0; k < kBlk; ++k) o[16 * k] = acc[0][k][q];
          if (c16 == 0)
            *reinterpret_cast<f32x2_t*>(a.ws_ml + (base + row) * 2) = f32x2_t{refq, l[0][q]};
        }
      });
      return;
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    pa::static_for<0, 4>([&](auto Q) {
      constexpr int q = decltype(Q)::value;
      const int row = 4 * jr + q;
      const int32_t ti = w0 + r * TP + row / GP, g = row % GP;
      if (ti < w1 && g < G) {
        const float inv = 1.f / l[r][q];
        uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) +
                        ((int64_t)(it.qs + ti) * H_q + kvh * G + g) * D + c16;
#pragma unroll
        for (int k = 0; k < kBlk / 2; ++k) {
          // columns 32 k + c and 32 k + 16 + c (lanes c of a row: 32 bytes each)
          const uint32_t pk = pa::pack2<E>(acc[r][2 * k][q] * inv, acc[r][2 * k + 1][q] * inv);
          dst[32 * k] = static_cast<uint16_t>(pk);
          dst[32 * k + 16] = static_cast<uint16_t>(pk >> 16);
        }
      }
    });
  }
}

// Combines the pieces of a split query block: workgroup f runs only if it
// holds piece 0 of a query block cut into S > 1 pieces, whose pieces are
// the workgroups f, f + H_kv, ..., f + (S - 1) H_kv of the attention grid.
// Thread t merges row t / 4 of the workgroup's rows, columns
// (t % 4) * D/4 .. + D/4:  M = max_s m_s,  out = sum_s 2^(m_s - M) o_s /
// sum_s 2^(m_s - M) l_s, rounded once to the output format.
template <int E, int D, int GP>
__global__ void __launch_bounds__(kThreads) prefill_merge_kernel(PrefillArgs a) {
  constexpr int TP = 16 / GP, QT = kNW * TP;
  constexpr int C = D / 4, NC = C / 4;  // columns per thread, as float4 chunks
  extern __shared__ __attribute__((aligned(16))) char smem[];
  Item it;
  if (!locate_item<QT, true>(a, smem, it)) return;
  if (it.S <= 1 || it.s != 0) return;
  const int32_t H_kv = a.pool.H_kv;
  if ((int64_t)blockIdx.x + (int64_t)(it.S - 1) * H_kv >= gridDim.x) return;  // malformed snapshot
  const int row = threadIdx.x >> 2, part = threadIdx.x & 3;
  const int rr = row & 15;
  const int32_t ti = it.i0 + (row >> 4) * TP + rr / GP, g = rr % GP;
  if (ti >= it.i1 || g >= a.G) return;
  float M = -3.0e38f;
  for (int32_t s = 0; s < it.S; ++s) {
    const int64_t slot = ((int64_t)blockIdx.x + (int64_t)s * H_kv) * kPieceRows + row;
    M = fmaxf(M, a.ws_ml[slot * 2]);
  }
  floatx4_t o[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) o[c] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  float l = 0.f;
  for (int32_t s = 0; s < it.S; ++s) {
    const int64_t slot = ((int64_t)blockIdx.x + (int64_t)s * H_kv) * kPieceRows + row;
    const f32x2_t ml = *reinterpret_cast<const f32x2_t*>(a.ws_ml + slot * 2);
    const float w = __builtin_amdgcn_exp2f(ml[0] - M);  // 0 for a piece with no keys here
    l = fmaf(w, ml[1], l);
    const floatx4_t* src = reinterpret_cast<const floatx4_t*>(a.ws_o + slot * D + part * C);
#pragma unroll
    for (int c = 0; c < NC; ++c) o[c] += w * src[c];
  }
  const float inv = 1.f / l;
  const int32_t H_q = H_kv * a.G;
  uint32_t* dst = reinterpret_cast<uint32_t*>(
      reinterpret_cast<char*>(a.out) +
      (((int64_t)(it.qs + ti) * H_q + it.kvh * a.G + g) * D + part * C) * 2);
#pragma unroll
  for (int c = 0; c < NC; c += 2) {
    const floatx4_t x = o[c] * inv, y = o[c + 1] * inv;
    *reinterpret_cast<u32x4_t*>(dst + 2 * c) =
        u32x4_t{pa::pack2<E>(x[0], x[1]), pa::pack2<E>(x[2], x[3]), pa::pack2<E>(y[0], y[1]),
                pa::pack2<E>(y[2], y[3])};
  }
}

template <int E, int D, int GP, int R, bool kSplit = false>
pa_status launch_r(const PrefillArgs& a, int64_t items, hipStream_t s) {
  auto kern = prefill_kernel<E, D, GP, R, kSplit>;
  const size_t lds = (size_t)header_bytes(a.B, kSplit) + 2 * TileGeo<D>::kStage;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess)
      return pa::fail(PA_ERR_DEVICE, "pa_prefill: LDS attribute: %s", hipGetErrorString(e));
  }
  hipLaunchKernelGGL(kern, dim3((uint32_t)items), dim3(kThreads), lds, s, a);
  if constexpr (kSplit)
    hipLaunchKernelGGL((prefill_merge_kernel<E, D, GP>), dim3((uint32_t)items), dim3(kThreads),
                       (size_t)header_bytes(a.B, true), s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pa::fail(PA_ERR_DEVICE, "pa_prefill: %s", hipGetErrorString(e));
  return PA_OK;
}

// Work items for R row blocks per wave: at most ceil(T / QT) + B query
// blocks per KV head (QT = 4 waves x R x 16 / GP tokens).
inline int64_t prefill_items(int32_t T, int32_t B, int32_t H_kv, int GP, int R) {
  const int64_t QT = (int64_t)kNW * R * (16 / GP);
  return (((int64_t)T + QT - 1) / QT + B) * H_kv;
}

inline int group_pad(int32_t G) { return G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : G <= 8 ? 8 : 16; }

inline size_t align_up(size_t x, size_t m) { return (x + m - 1) / m * m; }

// How pa_prefill_split runs a call of this shape, from host-known sizes
// only.  With at most kSplitMaxItems items of the one-row-block kernel (too
// few to keep every CU busy through the longest query blocks), query
// blocks are cut along the keys into pieces of key_tiles tiles: at least
// kMinKeyTiles, and enough that the grid stays near kSplitGrid workgroups.
// The grid bounds the pieces from above: every query block of the item
// bound taken as seeing all ceil(max_blocks * block_size / 32) key tiles.
// Each piece pays a fixed start (snapshot, query rows, the first tiles'
// loads), and so does each workgroup past the real pieces, so pieces stay
// long.  Measured on the worked batch (last N tokens of each sequence): N =
// 64 took 51 us split against 91 us whole, N = 128 68 against 94 (pieces of
// 48 tiles; 4-16 tile pieces were up to 4x slower), while N = 256 (928
// items) took 100 us whole and 109-115 us split.  The piece length can be
// set with pa_set_tuning(PA_TUNE_PREFILL_KEY_TILES, n).
struct SplitPlan {
  bool split;
  int32_t key_tiles;
  int64_t grid;
  size_t o_bytes, ws_bytes;
};
constexpr int64_t kSplitMaxItems = 640;
constexpr int64_t kMinKeyTiles = 48;
constexpr int64_t kSplitGrid = 1536;

SplitPlan split_plan(const pa_cache_desc* d, int32_t B, int32_t H_q, int32_t T, int32_t maxb) {
  SplitPlan p{false, 0, 0, 0, 0};
  if (B <= 0 || T <= 0 || maxb < 1) return p;
  const int32_t H_kv = d->num_kv_heads;
  const int GP = group_pad(H_q / H_kv);
  const int64_t items1 = prefill_items(T, B, H_kv, GP, 1);
  if (items1 > kSplitMaxItems || prefill_items(T, B, H_kv, GP, 2) >= kMinItemsR2) return p;
  const int64_t maxtiles = ((int64_t)maxb * d->block_size + kKT - 1) / kKT;
  int64_t kt = std::max<int64_t>(kMinKeyTiles, (maxtiles * items1 + kSplitGrid - 1) / kSplitGrid);
  if (const int32_t x = pa::tuning(PA_TUNE_PREFILL_KEY_TILES); x >= 1) kt = x;
  const int64_t S = (maxtiles + kt - 1) / kt;
  if (S <= 1 || items1 * S >= (1ll << 31)) return p;
  p.split = true;
  p.key_tiles = (int32_t)kt;
  p.grid = items1 * S;
  p.o_bytes = align_up((size_t)p.grid * kPieceRows * d->head_dim * sizeof(float), 256);
  p.ws_bytes = p.o_bytes + align_up((size_t)p.grid * kPieceRows * 2 * sizeof(float), 256);
  return p;
}

template <int E, int D, int GP>
pa_status launch(const PrefillArgs& a, const SplitPlan& plan, hipStream_t s) {
  const int64_t items1 = prefill_items(a.T, a.B, a.pool.H_kv, GP, 1);
  const int64_t items2 = prefill_items(a.T, a.B, a.pool.H_kv, GP, 2);
  if (items1 >= (1ll << 31))  // the kernel numbers items in int32
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_prefill: too many query blocks");
  if (plan.split) return launch_r<E, D, GP, 1, true>(a, plan.grid, s);
  if (items2 >= kMinItemsR2) return launch_r<E, D, GP, 2>(a, items2, s);
  return launch_r<E, D, GP, 1>(a, items1, s);
}

template <int E, int D>
pa_status dispatch_g(const PrefillArgs& a, const SplitPlan& plan, hipStream_t s) {
  if (a.G <= 1) return launch<E, D, 1>(a, plan, s);
  if (a.G <= 2) return launch<E, D, 2>(a, plan, s);
  if (a.G <= 4) return launch<E, D, 4>(a, plan, s);
  if (a.G <= 8) return launch<E, D, 8>(a, plan, s);
  return launch<E, D, 16>(a, plan, s);
}

// Checks the arguments shared by pa_prefill and pa_prefill_split and fills
// the kernel arguments; *nothing is set when the call has no work.
pa_status prefill_args(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* context_lens, const int32_t* query_start, int32_t num_seqs,
                       int32_t num_query_tokens, int32_t block_size, float scale, void* out,
                       int32_t num_q_heads, const pa_cache_desc* desc, PrefillArgs& a,
                       bool* nothing) {
  *nothing = false;
  pa_status st = pa_supported(desc, num_q_heads);
  if (st != PA_OK) return st;
  if (desc->dtype != PA_BF16 && desc->dtype != PA_F16)
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_prefill: 16-bit (bf16 or fp16) pools only");
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
  if ((int64_t)desc->num_blocks * desc->num_kv_heads * block_size > INT32_MAX)
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_prefill: pool of more than 2^31 rows per pool");
  if (num_seqs == 0 || num_query_tokens == 0) {
    *nothing = true;
    return PA_OK;
  }
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start || !out)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (!pa::aligned(q, 16) || !pa::aligned(k_cache, 16) || !pa::aligned(v_cache, 16) ||
      !pa::aligned(out, 16) || !pa::aligned(block_tables, 4) || !pa::aligned(context_lens, 4) ||
      !pa::aligned(query_start, 4))
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "misaligned pointer");
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
  a.key_tiles = 0;
  a.ws_o = nullptr;
  a.ws_ml = nullptr;
  return PA_OK;
}

pa_status run(const PrefillArgs& a, const SplitPlan& plan, const pa_cache_desc* desc,
              void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const bool d128 = desc->head_dim == 128;
  if (desc->dtype == PA_F16)
    return d128 ? dispatch_g<2, 128>(a, plan, s) : dispatch_g<2, 64>(a, plan, s);
  return d128 ? dispatch_g<1, 128>(a, plan, s) : dispatch_g<1, 64>(a, plan, s);
}

}  // namespace

extern "C" {

pa_status pa_prefill(const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, const int32_t* query_start, int32_t num_seqs,
                     int32_t num_query_tokens, int32_t block_size, float scale, void* out,
                     int32_t num_q_heads, const pa_cache_desc* desc, void* stream) {
  PrefillArgs a;
  bool nothing;
  pa_status st = prefill_args(q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                              context_lens, query_start, num_seqs, num_query_tokens, block_size,
                              scale, out, num_q_heads, desc, a, &nothing);
  if (st != PA_OK || nothing) return st;
  return run(a, SplitPlan{false, 0, 0, 0, 0}, desc, stream);
}

pa_status pa_prefill_split_workspace_size(const pa_cache_desc* desc, int32_t num_seqs,
                                          int32_t num_q_heads, int32_t num_query_tokens,
                                          int32_t max_blocks_per_seq, size_t* bytes) {
  pa_status st = pa_supported(desc, num_q_heads);
  if (st != PA_OK) return st;
  if (!bytes) return pa::fail(PA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (num_seqs < 0 || num_query_tokens < 0 || max_blocks_per_seq < 1)
    return pa::fail(PA_ERR_INVALID_ARGUMENT, "num_seqs %d / num_query_tokens %d / "
                    "max_blocks_per_seq %d", num_seqs, num_query_tokens, max_blocks_per_seq);
  *bytes = split_plan(desc, num_seqs, num_q_heads, num_query_tokens, max_blocks_per_seq).ws_bytes;
  return PA_OK;
}

pa_status pa_prefill_split(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, const int32_t* query_start,
                           int32_t num_seqs, int32_t num_query_tokens, int32_t block_size,
                           float scale, void* out, int32_t num_q_heads,
                           const pa_cache_desc* desc, void* workspace, size_t workspace_bytes,
                           void* stream) {
  PrefillArgs a;
  bool nothing;
  pa_status st = prefill_args(q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                              context_lens, query_start, num_seqs, num_query_tokens, block_size,
                              scale, out, num_q_heads, desc, a, &nothing);
  if (st != PA_OK || nothing) return st;
  const SplitPlan plan =
      split_plan(desc, num_seqs, num_q_heads, num_query_tokens, max_blocks_per_seq);
  if (plan.split) {
    if (!workspace) return pa::fail(PA_ERR_INVALID_ARGUMENT, "NULL workspace");
    if (!pa::aligned(workspace, 256))
      return pa::fail(PA_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
    if (workspace_bytes < plan.ws_bytes)
      return pa::fail(PA_ERR_INVALID_ARGUMENT, "workspace %zu bytes < %zu needed",
                      workspace_bytes, plan.ws_bytes);
    a.key_tiles = plan.key_tiles;
    a.ws_o = reinterpret_cast<float*>(workspace);
    a.ws_ml = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + plan.o_bytes);
  }
  return run(a, plan, desc, stream);
}

}  // extern "C"
