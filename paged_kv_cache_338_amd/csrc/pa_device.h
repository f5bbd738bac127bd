// Device helpers shared by the library's HIP translation units (gfx950,
// wave64).  Not installed.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>
#include <utility>

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// DPP row_newbcast: every lane of a 16-lane row reads lane N of that row.
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
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

// bf16 halves of a packed word, widened exactly to fp32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __builtin_bit_cast(float, w & 0xFFFF0000u);
}

// fp32 -> bf16 with round-to-nearest-even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// ---- 16-bit element kinds.  E is the pool's element kind: 0 = fp32,
// 1 = bf16, 2 = fp16 (the pa_dtype codes).  The helpers below pick the MFMA
// instruction, the packing and the rounding of a 16-bit kind; for E = 1
// they are exactly the bf16 operations.
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef short s16x4_v __attribute__((ext_vector_type(4)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));

// 16x16x32 MFMA: a, b hold 8 elements each (4 words).
template <int E>
__device__ __forceinline__ floatx4_t mfma_k32(u32x4_t a, u32x4_t b, floatx4_t c) {
  static_assert(E == 1 || E == 2, "16-bit kinds only");
  if constexpr (E == 2)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// 16x16x16 MFMA: a, b hold 4 elements each (2 words, as one 64-bit value).
template <int E>
__device__ __forceinline__ floatx4_t mfma_k16(uint64_t a, uint64_t b, floatx4_t c) {
  static_assert(E == 1 || E == 2, "16-bit kinds only");
  if constexpr (E == 2)
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                 __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_v, a),
                                                     __builtin_bit_cast(s16x4_v, b), c, 0, 0, 0);
}

// Two fp32 values rounded (to nearest even) and packed, lo in bits 0..15.
template <int E>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const f32x2_v v = {lo, hi};
  if constexpr (E == 2) return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
  else return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_v));
}

// The 16-bit halves of a packed word, widened exactly to fp32.
template <int E>
__device__ __forceinline__ float lo16(uint32_t w) {
  if constexpr (E == 2)
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xFFFFu)));
  else return __builtin_bit_cast(float, w << 16);
}
template <int E>
__device__ __forceinline__ float hi16(uint32_t w) {
  if constexpr (E == 2)
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
  else return __builtin_bit_cast(float, w & 0xFFFF0000u);
}

// fp32 -> the 16-bit kind, round to nearest even.
template <int E>
__device__ __forceinline__ uint16_t round16(float x) {
  if constexpr (E == 2) return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
  else {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
  }
}

// Two 1.0 values of the kind, packed.
template <int E>
constexpr uint32_t kOnes2 = E == 2 ? 0x3C003C00u : 0x3F803F80u;

// Workgroup barrier that orders LDS only: global loads still in flight are
// not drained (unlike __syncthreads(), a full workgroup fence).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Reductions over the four 16-lane rows (lanes l, l^16, l^32, l^48) with
// the gfx950 row-swap permutes: no LDS traffic, so they do not share the
// LGKM counter with scalar loads in flight.  permlane32_swap of x with
// itself leaves {x[l], x[l^32]} in its two results on every lane, and
// permlane16_swap leaves {x[l], x[l^16]}.
__device__ __forceinline__ float rows_sum(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float y = as_float(a[0]) + as_float(a[1]);
  const uint32_t w = __builtin_bit_cast(uint32_t, y);
  const auto b = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return as_float(b[0]) + as_float(b[1]);
}
__device__ __forceinline__ float rows_max(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float y = fmaxf(as_float(a[0]), as_float(a[1]));
  const uint32_t w = __builtin_bit_cast(uint32_t, y);
  const auto b = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return fmaxf(as_float(b[0]), as_float(b[1]));
}

// Lane 16j + c receives x from lane 4j + Q (row j picks its own source;
// the sources lie in lanes 0..15).  Read through SGPRs, without LDS.
template <int Q>
__device__ __forceinline__ float pick_row_quad(float x, int jr) {
  const int xi = __builtin_bit_cast(int, x);
  const float s0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, Q));
  const float s1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 4 + Q));
  const float s2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 8 + Q));
  const float s3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 12 + Q));
  return jr == 0 ? s0 : (jr == 1 ? s1 : (jr == 2 ? s2 : s3));
}

// Integer DPP move: lanes whose source is outside the row (or rows left out
// of RowMask) read 0.
template <int Ctrl, int RowMask = 0xF>
__device__ __forceinline__ int dpp_or_zero(int x) {
  return __builtin_amdgcn_update_dpp(0, x, Ctrl, RowMask, 0xF, true);
}

// Inclusive prefix sum over the 64 lanes with DPP only (no LDS): shifts by
// 1, 2, 4 and 8 within each 16-lane row, then row_bcast:15 adds row 0's
// total to row 1 and row 2's to row 3, and row_bcast:31 adds the total of
// rows 0-1 to rows 2-3.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp_or_zero<0x111>(v);       // row_shr:1
  v += dpp_or_zero<0x112>(v);       // row_shr:2
  v += dpp_or_zero<0x114>(v);       // row_shr:4
  v += dpp_or_zero<0x118>(v);       // row_shr:8
  v += dpp_or_zero<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_or_zero<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

}  // namespace pa
