// Measurement kernels for the decode's cost floor (libpa_floor.so, loaded by
// the benchmark only; not part of the decode path).
//
// Each one does a part of what a paged decode call must do and nothing else,
// so the time of a decode call can be set against the time of its parts on
// the same GPU and pools:
//   * pa_floor_read_tiles: read every (block, KV head) tile a decode reads,
//     K and V, from a precomputed list of byte offsets (no table walk, no
//     length arithmetic, no attention arithmetic, no partial results);
//   * pa_floor_read_contiguous: read the same number of bytes as one
//     contiguous range per pool;
//   * pa_floor_empty: a launch that does nothing (the per-launch cost).
// Loads are non-temporal, as the decode's K/V loads.  Loaded words are
// folded by XOR into a value stored only when it equals a caller-chosen
// number, so the loads cannot be dropped and almost nothing is written.
// Every entry point returns a hipError_t value.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTileBytes = 4096;  // 16 tokens x 128 values x 2 bytes

// Non-temporal, as the decode's K/V loads: each byte is read once per launch.
__device__ inline u32x4 ld16(const char* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ inline void sink_if(u32x4 acc, uint32_t magic, uint32_t* sink) {
  const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (x == magic) sink[blockIdx.x * kThreads + threadIdx.x] = x;
}

// Each wave takes a contiguous share of the tile list (the decode's split of
// its units); per tile each lane reads 64 bytes of K and 64 of V, two tiles
// in flight.
__global__ __launch_bounds__(kThreads) void read_tiles_kernel(const char* k, const char* v,
                                                              const int64_t* offs, int32_t n,
                                                              uint32_t magic, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * kWaves;
  const int64_t gw = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int64_t u1 = n * (gw + 1) / waves;
  int64_t u = n * gw / waves;
  u32x4 acc = {0, 0, 0, 0};
  for (; u + 1 < u1; u += 2) {
    const int64_t o0 = offs[u] + lane * 16, o1 = offs[u + 1] + lane * 16;
    u32x4 r[16];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      r[c] = ld16(k + o0 + c * 1024);
      r[4 + c] = ld16(v + o0 + c * 1024);
      r[8 + c] = ld16(k + o1 + c * 1024);
      r[12 + c] = ld16(v + o1 + c * 1024);
    }
#pragma unroll
    for (int c = 0; c < 16; ++c) acc ^= r[c];
  }
  if (u < u1) {
    const int64_t o0 = offs[u] + lane * 16;
#pragma unroll
    for (int c = 0; c < 4; ++c) acc ^= ld16(k + o0 + c * 1024) ^ ld16(v + o0 + c * 1024);
  }
  sink_if(acc, magic, sink);
}

// Grid-stride read of [0, bytes) of each of two buffers, 16 bytes per lane,
// four loads of each buffer in flight.
__global__ __launch_bounds__(kThreads) void read_contiguous_kernel(const char* a, const char* b,
                                                                   int64_t bytes, uint32_t magic,
                                                                   uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * kThreads * 16;
  int64_t i = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 16;
  u32x4 acc = {0, 0, 0, 0};
  for (; i + 3 * stride < bytes; i += 4 * stride) {
    u32x4 r[8];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      r[c] = ld16(a + i + c * stride);
      r[4 + c] = ld16(b + i + c * stride);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) acc ^= r[c];
  }
  for (; i < bytes; i += stride) acc ^= ld16(a + i) ^ ld16(b + i);
  sink_if(acc, magic, sink);
}

__global__ __launch_bounds__(kThreads) void empty_kernel() {}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

extern "C" {

// k, v: device pools; offs: device int64[n], byte offsets of 4096-byte tiles
// (16-byte aligned, each tile inside both pools: the caller checks);
// sink: device uint32[wgs * 256].
int pa_floor_read_tiles(const void* k, const void* v, const int64_t* offs, int32_t n,
                        int32_t wgs, uint32_t magic, uint32_t* sink, void* stream) {
  if (!k || !v || !offs || !sink || n < 0 || wgs < 1 || wgs > 65536 || !aligned16(k) ||
      !aligned16(v))
    return hipErrorInvalidValue;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(read_tiles_kernel, dim3(wgs), dim3(kThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const char*>(k),
                     static_cast<const char*>(v), offs, n, magic, sink);
  return hipGetLastError();
}

// a, b: device buffers of at least `bytes` bytes each (a multiple of 16).
int pa_floor_read_contiguous(const void* a, const void* b, int64_t bytes, int32_t wgs,
                             uint32_t magic, uint32_t* sink, void* stream) {
  if (!a || !b || !sink || bytes < 0 || bytes % 16 || wgs < 1 || wgs > 65536 || !aligned16(a) ||
      !aligned16(b))
    return hipErrorInvalidValue;
  if (bytes == 0) return hipSuccess;
  hipLaunchKernelGGL(read_contiguous_kernel, dim3(wgs), dim3(kThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const char*>(a),
                     static_cast<const char*>(b), bytes, magic, sink);
  return hipGetLastError();
}

int pa_floor_empty(int32_t wgs, void* stream) {
  if (wgs < 1 || wgs > 65536) return hipErrorInvalidValue;
  hipLaunchKernelGGL(empty_kernel, dim3(wgs), dim3(kThreads), 0,
                     reinterpret_cast<hipStream_t>(stream));
  return hipGetLastError();
}

int pa_floor_tile_bytes() { return kTileBytes; }

}  // extern "C"
