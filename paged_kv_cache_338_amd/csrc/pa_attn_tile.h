// K/V tile loading and the per-tile MFMA attention step shared by the
// decode and prefill kernels (gfx950 / CDNA4, wave64).  Not installed.
//
// A tile is 16 consecutive tokens of one (sequence, KV head): 16 K rows and
// 16 V rows of the pool's [num_blocks][H_kv][bs][D] layout, found through
// the sequence's block table (token t is row t % bs of physical block
// table[t / bs]).
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "pa_device.h"

namespace pa {

constexpr int kTile = 16;  // tokens per tile (one MFMA row block)

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// The pool pair as a kernel sees it.
struct KvPool {
  const void* k_cache;
  const void* v_cache;
  int32_t num_blocks;
  int32_t H_kv;
  int32_t log2_bs;
};

template <bool k16, int D>
struct Geometry {
  static constexpr int kElem = k16 ? 2 : 4;
  static constexpr int kRowBytes = D * kElem;
  static constexpr int kKPieces = kRowBytes / 64;     // 16-byte K pieces per lane per tile
  static constexpr int kVWords = kRowBytes / 16 / 4;  // 32-bit words of V per lane per token
  static constexpr int kCols = D / 16;                // output columns per lane
  static constexpr int kQRegs = k16 ? kKPieces : 1;  // query as 16-bit MFMA operand
  static constexpr int kQF32 = k16 ? 1 : kKPieces * 4;
  static_assert(kRowBytes % 64 == 0, "row must be a multiple of 64 bytes");
};

template <bool k16, int D>
struct TileRegs {
  using Geo = Geometry<k16, D>;
  u32x4_t k[Geo::kKPieces];
  uint32_t v[4][Geo::kVWords];
};

__device__ __forceinline__ int32_t uni(int32_t x) { return __builtin_amdgcn_readfirstlane(x); }

// A wave-uniform pointer, moved to SGPRs.
__device__ __forceinline__ char* uniform_ptr(const char* p) {
  const uint64_t x = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x >> 32));
  return reinterpret_cast<char*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Cache-policy operand of the buffer loads: non-temporal (the loaded lines
// are the first the caches give up), for data read once per launch.
constexpr int kNonTemporal = 2;

// Buffer-resource word 3 for raw dword loads on gfx9-family parts (32-bit
// data format; a zero format would make every load return zero).
constexpr int32_t kRsrcWord3 = 0x00020000;

// Issues the K/V loads of tile t of a segment (KV head kvh) whose 16 rows
// lie in physical block `phys` (blocks of >= 16 tokens).  The rows are read
// through a buffer resource spanning exactly them; pipeline padding
// (`valid` false) gets a zero-length resource, so its loads return zeros
// without touching memory.  Rows past the context length stay inside the
// block and are masked when consumed.
// kNT: non-temporal loads.
template <bool k16, int D, bool kNT = false>
__device__ __forceinline__ void issue_tile(TileRegs<k16, D>& r, const KvPool& a,
                                           int32_t phys, int32_t t, int32_t kvh, int lane,
                                           bool valid) {
  constexpr int kAux = kNT ? kNonTemporal : 0;
  using Geo = Geometry<k16, D>;
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
    r.k[p] = __builtin_bit_cast(
        u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, ko + p * 64, 0, kAux));
  const int32_t vo = (jr * 4) * Geo::kRowBytes + c16 * (Geo::kVWords * 4);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int h = 0; h < Geo::kVWords; h += 4) {
      if constexpr (Geo::kVWords >= 4) {
        const u32x4_t x = __builtin_bit_cast(
            u32x4_t,
            __builtin_amdgcn_raw_buffer_load_b128(rv, vo + q * Geo::kRowBytes + h * 4, 0, kAux));
        r.v[q][h + 0] = x[0];
        r.v[q][h + 1] = x[1];
        r.v[q][h + 2] = x[2];
        r.v[q][h + 3] = x[3];
      } else {
        const uint2 x = __builtin_bit_cast(
            uint2, __builtin_amdgcn_raw_buffer_load_b64(rv, vo + q * Geo::kRowBytes, 0, kAux));
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
//
// new_row >= 0: row new_row of the tile is read from nk / nv (the first byte
// of the new token's K and V rows) instead of the pools (see
// issue_tile_with_row).
template <bool k16, int D, bool kNT = false>
__device__ __forceinline__ void issue_tile_small(TileRegs<k16, D>& r, const KvPool& a,
                                                 int32_t phys_v, int32_t jl, int32_t t,
                                                 int32_t kvh, int32_t L, int nbt, int lane,
                                                 int32_t new_row = -1, const char* nk = nullptr,
                                                 const char* nv = nullptr) {
  using Geo = Geometry<k16, D>;
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
  // The pool addresses are formed in every lane before any lane takes the
  // new row instead: row_addr's shuffle reads other lanes, which must all be
  // active.
  const char* kc = row_addr(lane & 15, a.k_cache);
  const char* kp = (c16 == new_row ? nk : kc) + jr * 16;
  auto ld16 = [](const char* p) -> u32x4_t {
    if constexpr (kNT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    else return *reinterpret_cast<const u32x4_t*>(p);
  };
#pragma unroll
  for (int p = 0; p < Geo::kKPieces; ++p) r.k[p] = ld16(kp + p * 64);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const char* vc = row_addr(jr * 4 + q, a.v_cache);
    const char* vp = (jr * 4 + q == new_row ? nv : vc) + c16 * (Geo::kVWords * 4);
#pragma unroll
    for (int h = 0; h < Geo::kVWords; h += 4) {
      if constexpr (Geo::kVWords >= 4) {
        const u32x4_t x = ld16(vp + h * 4);
        r.v[q][h + 0] = x[0];
        r.v[q][h + 1] = x[1];
        r.v[q][h + 2] = x[2];
        r.v[q][h + 3] = x[3];
      } else {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        u32x2 x;
        if constexpr (kNT) x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(vp));
        else x = *reinterpret_cast<const u32x2*>(vp);
        r.v[q][0] = x[0];
        r.v[q][1] = x[1];
      }
    }
  }
}

// For the tile that holds a sequence's newest token (written to the pools
// by the same launch), after issue_tile: row new_row of the tile is loaded
// again, from the token's own K and V rows (nk, nv: their first bytes),
// into the lanes that hold that row, so the result does not depend on when
// the write lands.  Buffer loads like issue_tile's, so they return after
// the pool's loads into the same registers.
template <bool k16, int D>
__device__ __forceinline__ void reload_new_row(TileRegs<k16, D>& r, int32_t new_row,
                                               const char* nk, const char* nv, int lane) {
  using Geo = Geometry<k16, D>;
  const int jr = lane >> 4, c16 = lane & 15;
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(nk), 0, Geo::kRowBytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(nv), 0, Geo::kRowBytes, kRsrcWord3);
  if (c16 == new_row) {
#pragma unroll
    for (int p = 0; p < Geo::kKPieces; ++p)
      r.k[p] = __builtin_bit_cast(u32x4_t,
                                  __builtin_amdgcn_raw_buffer_load_b128(rk, jr * 16 + p * 64, 0, 0));
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (jr * 4 + q == new_row) {
      const int32_t vo = c16 * (Geo::kVWords * 4);
#pragma unroll
      for (int h = 0; h < Geo::kVWords; h += 4) {
        if constexpr (Geo::kVWords >= 4) {
          const u32x4_t x = __builtin_bit_cast(
              u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, vo + h * 4, 0, 0));
          r.v[q][h + 0] = x[0];
          r.v[q][h + 1] = x[1];
          r.v[q][h + 2] = x[2];
          r.v[q][h + 3] = x[3];
        } else {
          const uint2 x = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rv, vo, 0, 0));
          r.v[q][0] = x.x;
          r.v[q][1] = x.y;
        }
      }
    }
  }
}

// Consumes one tile: logits by MFMA, online softmax per 16-lane row, P*V.
// t0 = first token of the tile within its sequence, end = context length.


// Per-wave state over one piece, 16-bit pools (P*V by MFMA).
//  ref: lane 16j + g: reference max of head g (log2 units), equal in all rows.
//  l:   lane 16j + c, register r: sum of the (16-bit-rounded) weights of head
//       4j + r, equal in every column c (an MFMA of P against ones).
//  acc[blk]: lane 16j + c, register r: unnormalised output of head 4j + r at
//       column (D/16)*c + blk.
template <int D>
struct MfmaState {
  static constexpr int kBlk = D / 16;
  float ref;
  floatx4_t l;
  floatx4_t acc[kBlk];

  __device__ __forceinline__ void reset() {
    ref = -3.0e38f;
    l = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < kBlk; ++b) acc[b] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  }
};

// Consumes one tile (16-bit kind E): logits S = K q^T by MFMA (lane 16j + c holds
// query row c, tokens 4j..4j+3); weights p = 2^(x - ref) against a reference
// max that is raised (and the accumulators rescaled) only when a logit
// exceeds it by more than 2^8, so the common tile needs no cross-lane
// reduction; then O += P V by MFMA with P (heads x tokens) exactly where the
// logits are and V (tokens x columns) made from the lane's own V rows, and
// l += P 1 by one more MFMA.  Only a tail tile (past the context length)
// masks: its logits there become -inf (weight 0) and its V rows there
// become 0, so garbage or NaN in unused slots cannot leak.  Heads >= G have
// zero query rows; their rows are computed and never stored.
// kTail: key t of the tile is masked for the lane's query row when t > lim
// (lim may differ per lane: a causal limit), and V rows at or past vend (the
// tokens in the cache) are zeroed.
template <int E, int D, bool kTail>
__device__ __forceinline__ void consume_tile_mfma_impl(MfmaState<D>& st,
                                                       const TileRegs<true, D>& r,
                                                       const u32x4_t* qf, float scale_log2,
                                                       int32_t t0, int32_t lim, int32_t vend,
                                                       int lane) {
  using Geo = Geometry<true, D>;
  constexpr int kBlk = MfmaState<D>::kBlk;
  const int jr = lane >> 4;
  floatx4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < Geo::kKPieces; ++p) s = mfma_k32<E>(r.k[p], qf[p], s);
  float x[4];
  bool hi = false;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    x[q] = s[q] * scale_log2;
    if constexpr (kTail)
      if (t0 + jr * 4 + q > lim) x[q] = -INFINITY;
    hi = hi || x[q] > st.ref + 8.f;
  }
  if (__ballot(hi) != 0) {  // uniform: raise the reference
    float mt = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mt = pa::rows_max(mt);
    const float nref = fmaxf(st.ref, mt);
    const float f = __builtin_amdgcn_exp2f(st.ref - nref);
    st.ref = nref;
    pa::static_for<0, 4>([&](auto Q) {
      constexpr int q = decltype(Q)::value;
      const float fr = pa::pick_row_quad<q>(f, jr);  // head 4j + q
      st.l[q] *= fr;
#pragma unroll
      for (int b = 0; b < kBlk; ++b) st.acc[b][q] *= fr;
    });
  }
  const uint32_t a01 = pack2<E>(__builtin_amdgcn_exp2f(x[0] - st.ref),
                                 __builtin_amdgcn_exp2f(x[1] - st.ref));
  const uint32_t a23 = pack2<E>(__builtin_amdgcn_exp2f(x[2] - st.ref),
                                 __builtin_amdgcn_exp2f(x[3] - st.ref));
  const uint64_t pa_ = (uint64_t)a01 | ((uint64_t)a23 << 32);
  uint32_t m01 = 0xFFFFFFFFu, m23 = 0xFFFFFFFFu;
  if constexpr (kTail) {
    const int32_t row0 = t0 + jr * 4;
    m01 = (row0 + 0 < vend ? 0x0000FFFFu : 0u) | (row0 + 1 < vend ? 0xFFFF0000u : 0u);
    m23 = (row0 + 2 < vend ? 0x0000FFFFu : 0u) | (row0 + 3 < vend ? 0xFFFF0000u : 0u);
  }
#pragma unroll
  for (int b = 0; b < kBlk; ++b) {
    const int w = b >> 1;
    const uint32_t sel = (b & 1) ? 0x07060302u : 0x05040100u;
    uint32_t v01 = __builtin_amdgcn_perm(r.v[1][w], r.v[0][w], sel);
    uint32_t v23 = __builtin_amdgcn_perm(r.v[3][w], r.v[2][w], sel);
    if constexpr (kTail) {
      v01 &= m01;
      v23 &= m23;
    }
    st.acc[b] = mfma_k16<E>(pa_, (uint64_t)v01 | ((uint64_t)v23 << 32), st.acc[b]);
  }
  constexpr uint64_t ones = (uint64_t)kOnes2<E> | ((uint64_t)kOnes2<E> << 32);  // 1.0 x 4
  st.l = mfma_k16<E>(pa_, ones, st.l);
}

}  // namespace pa
