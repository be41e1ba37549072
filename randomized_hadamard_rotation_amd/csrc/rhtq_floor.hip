// Streaming floor of a launch shape (include/rhtq_floor.h): a measurement aid beside the
// method, not part of it.  The kernel moves the bytes of a per-row 4-bit forward call with
// the forward kernel's grid and workgroup shape and the same access pattern, and computes
// nothing but XOR folds of the loaded words:
//
//  - wave h of a row's workgroup reads the half h of the row as 512-element fragments, lane l
//    loading the 16 bytes at element 512 f + 8 l of fragment f (non-temporal);
//  - per fragment it stores one 4-byte word per lane, the XOR of that lane's four loaded
//    words, at code byte (n/2) h + 256 f + 4 l of the row (the code bytes of those elements);
//  - scale word w of the row (w < scale_bytes_per_row / 4) is written by lane w & 63 of wave
//    w >> 6 as the XOR of the first and last loaded words of that lane.
//
// Rows are taken in grid-stride order; the next row's loads go out before the current row's
// stores, as in the persistent forward kernels.
#include "rhtq.h"
#include "rhtq_device.h"
#include "rhtq_floor.h"
#include "rhtq_internal.h"

namespace rhtq {
namespace {

// The XOR folds of one row's loaded words (wave h's half): one word per fragment, one scale word.
template <int N>
__device__ __forceinline__ void floor_fold(const uint4 (&raw)[N / 1024], uint32_t (&o)[N / 1024], uint32_t& sw) {
  constexpr int F = N / 1024;
#pragma unroll
  for (int f = 0; f < F; ++f) o[f] = raw[f].x ^ raw[f].y ^ raw[f].z ^ raw[f].w;
  sw = raw[0].x ^ raw[F - 1].w;
}

template <int N>
__device__ __forceinline__ void floor_write(const uint32_t (&o)[N / 1024], uint32_t sw, int64_t row, int h,
                                            int lane, uint8_t* __restrict__ packed, uint8_t* __restrict__ scales,
                                            int scale_words) {
  constexpr int F = N / 1024;
  uint8_t* p = packed + row * (N / 2) + (N / 4) * h + 4 * lane;
#pragma unroll
  for (int f = 0; f < F; ++f) st_stream(p + 256 * f, o[f]);
  const int w = 64 * h + lane;
  // plain store, as the forward kernels write their scales (a non-temporal store of a few
  // bytes per row, to lines shared with other workgroups, costs several microseconds here)
  if (w < scale_words) reinterpret_cast<uint32_t*>(scales)[row * scale_words + w] = sw;
}

// PERSISTENT = false: one row per workgroup (grid = rows).  PERSISTENT = true: rows in
// grid-stride order, the next row's loads issued between the current row's folds and stores.
template <int N, bool PERSISTENT>
__global__ __launch_bounds__(128) void floor_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                    uint8_t* __restrict__ packed, uint8_t* __restrict__ scales,
                                                    int scale_words) {
  constexpr int F = N / 1024;   // fragments of 512 in a wave's half row
  const int lane = threadIdx.x & 63, h = threadIdx.x >> 6;
  uint4 raw[F];
  auto load = [&](int64_t r) {
#pragma unroll
    for (int f = 0; f < F; ++f) raw[f] = ld_stream(x + r * N + (N / 2) * h + 512 * f + 8 * lane);
  };
  int64_t row = blockIdx.x;
  if (row >= rows) return;
  load(row);
  uint32_t o[F], sw;
  for (;;) {
    floor_fold<N>(raw, o, sw);
    const int64_t next = row + gridDim.x;
    const bool more = PERSISTENT && next < rows;
    if (more) load(next);
    floor_write<N>(o, sw, row, h, lane, packed, scales, scale_words);
    if (!more) break;
    row = next;
  }
}

template <int N, bool PERSISTENT>
hipError_t launch_floor(const void* x, int64_t rows, void* packed, void* scales, int scale_words, int64_t grid,
                        hipStream_t s) {
  hipLaunchKernelGGL((floor_kernel<N, PERSISTENT>), dim3((unsigned)grid), dim3(128), 0, s, static_cast<const uint16_t*>(x), rows,
                     static_cast<uint8_t*>(packed), static_cast<uint8_t*>(scales), scale_words);
  return hipGetLastError();
}

bool aligned_to(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace
}  // namespace rhtq

extern "C" int rhtq_stream_floor(const void* x, int64_t tokens, int32_t n, void* packed_out, void* scales_out,
                                 int32_t scale_bytes_per_row, rhtq_stream_t stream) {
  using namespace rhtq;
  if (tokens < 0) return RHTQ_EINVAL;
  if (scale_bytes_per_row < 4 || scale_bytes_per_row > 512 || scale_bytes_per_row % 4 != 0) return RHTQ_EINVAL;
  if (n != 4096 && n != 12288) return RHTQ_EUNSUPPORTED;
  if (tokens == 0) return RHTQ_OK;
  if (x == nullptr || packed_out == nullptr || scales_out == nullptr) return RHTQ_EINVAL;
  if (!aligned_to(x, 16) || !aligned_to(packed_out, 4) || !aligned_to(scales_out, 4)) return RHTQ_EINVAL;
  if (tokens > 0xFFFFFFFELL) return RHTQ_EINVAL;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int words = scale_bytes_per_row / 4;
  hipError_t e;
  if (n == 4096) {
    e = launch_floor<4096, false>(x, tokens, packed_out, scales_out, words, tokens, s);
  } else {
    e = launch_floor<12288, true>(x, tokens, packed_out, scales_out, words, fast12_grid(tokens), s);
  }
  return e == hipSuccess ? RHTQ_OK : RHTQ_EHIP;
}
